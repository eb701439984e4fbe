"""GPU W4A16 GEMM against the float64 oracle.

Bar: max |y_gpu - y_ref| <= 1e-2 * max |y_ref| over each output tensor, where
y_ref is the oracle's unrounded float64 product; exact special cases must be
bit-identical to the correctly rounded exact result.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import awq, gemm as ogemm, numerics
from gpu_util import (DEV, TORCH_DTYPE, bits_to_device, device_to_bits, int32_to_device, oracle_repack,
                      oracle_y, weights_to_device, whole_output_error, y_to_f64)

pytestmark = pytest.mark.gpu
TOL = ogemm.TOLERANCE


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def pack_on_gpu(w, ws):
    qw, qz, sc = weights_to_device(ws)
    return w.w4a16_repack(qw, qz, sc, ws.group_size)


def run(w, ws, packed, x_bits, path="auto", bias=None, stream=None):
    x = bits_to_device(x_bits, ws.dtype)
    y = w.w4a16_gemm_ex(x, packed, ws.N, ws.group_size, bias=bias, path=path, stream=stream)
    torch.cuda.synchronize()
    return y


WORKLOAD_CASES = [(name, M) for name, wl in synth.WORKLOADS.items() for M in wl.Ms]


@pytest.mark.parametrize("name,M", WORKLOAD_CASES, ids=[f"{n}-M{m}" for n, m in WORKLOAD_CASES])
def test_gemm_workloads(w, name, M):
    print(f"gemm workload {name} M={M}", flush=True)
    ws = synth.make(name)
    packed = pack_on_gpu(w, ws)
    y = run(w, ws, packed, ws.x_bits[M])
    got = y_to_f64(y, ws.dtype)
    # the whole [M, N] output, the oracle taken in column chunks for the wide head
    err, _ = whole_output_error(got, lambda cols: oracle_y(ws, ws.x_bits[M], cols))
    print(f"  max rel err over all {M} x {ws.N} outputs {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("M", list(range(1, 18)) + [24, 31, 32, 33, 63, 64, 65, 100, 128, 129, 200])
def test_gemm_m_sweep_auto(w, M):
    ws = synth.make_custom(500 + M, M, 1152, 272, "bf16", 128)   # 9 row blocks, 17 column blocks (ragged tile)
    packed = pack_on_gpu(w, ws)
    got = y_to_f64(run(w, ws, packed, ws.x_bits[M]), "bf16")
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[M])) <= TOL


@pytest.mark.parametrize("path", ["gemv", "mfma"])
@pytest.mark.parametrize("M", [1, 2, 4, 7, 8, 9, 15, 16])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_gemm_forced_paths(w, path, M, dtype):
    ws = synth.make_custom(900 + M, M, 6656, 48, dtype, 128)        # down-projection K, 52 row blocks
    packed = pack_on_gpu(w, ws)
    got = y_to_f64(run(w, ws, packed, ws.x_bits[M], path=path), dtype)
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[M])) <= TOL


def test_gemm_from_oracle_packed_buffer(w):
    # the GEMM alone, fed the oracle's packed bytes (no GPU repack involved)
    ws = synth.make_custom(41, 24, 1024, 512, "bf16", 128)
    packed = torch.from_numpy(oracle_repack(ws)).to(DEV)
    for path in ("gemv", "mfma"):
        M = 16 if path == "gemv" else 24
        xb = ws.x_bits[24][:M]
        got = y_to_f64(run(w, ws, packed, xb, path=path), "bf16")
        assert ogemm.max_rel_error(got, oracle_y(ws, xb)) <= TOL


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_one_hot_rows_are_exact(w, dtype, path):
    # x = e_k: y[m, :] = W[k_m, :] = (q - z) * s exactly, so the output must be the
    # correctly rounded weight row, bit for bit; pins the k <-> lane/slot mapping
    K, N, G = 512, 64, 128
    rng = np.random.default_rng(3)
    ws = synth.make_custom(3, 1, K, N, dtype, G)
    M = 16
    ks = rng.choice(K, size=M, replace=False)
    x = np.zeros((M, K), dtype=np.float64)
    x[np.arange(M), ks] = 1.0
    xb = numerics.f64_to_half_bits_rne(x, dtype)
    packed = pack_on_gpu(w, ws)
    got = device_to_bits(run(w, ws, packed, xb, path=path))
    ref = oracle_y(ws, xb)
    assert np.array_equal(got, numerics.f64_to_half_bits_rne(ref, dtype))


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_small_integer_case_is_exact(w, path):
    # x in {-1, 0, 1}, s = 2^-6: every product and partial sum is exact in fp32,
    # so any summation order gives the exact result and the output is RNE(y)
    K, N, G, M = 1024, 96, 128, 12
    rng = np.random.default_rng(12)
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    Z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    ws = synth.make_custom(12, M, K, N, "bf16", G)
    ws.qweight, ws.qzeros = awq.pack_awq(Q), awq.pack_awq(Z)
    ws.scale_bits = np.full((K // G, N), 0x3C80, np.uint16)        # bf16 2^-6
    xb = numerics.f64_to_half_bits_rne(rng.integers(-1, 2, (M, K)).astype(np.float64), "bf16")
    packed = pack_on_gpu(w, ws)
    got = device_to_bits(run(w, ws, packed, xb, path=path))
    assert np.array_equal(got, numerics.f64_to_half_bits_rne(oracle_y(ws, xb), "bf16"))


# More tiles than compute units on a tile whose LDS holds one workgroup per CU: the
# grid is one workgroup per CU, each taking a tile per round and copying the next
# tile's first k block while it writes the current output. Ragged rows, a last half
# block of columns, N tiles that are not a multiple of 8 (ids without a tile), bias.
@pytest.mark.parametrize("M,K,N,dtype,with_bias", [
    (200, 1024, 32776, "bf16", True),     # 128 x 128 tiles, 2 x 257
    (300, 256, 36872, "fp16", False),     # 64 x 256 tiles, 5 x 145
    (1000, 256, 8200, "bf16", True),      # 128 x 128 tiles, 8 x 65
])
def test_gemm_more_tiles_than_cus(w, M, K, N, dtype, with_bias):
    print(f"gemm M={M} K={K} N={N} {dtype} bias={with_bias}", flush=True)
    ws = synth.make_custom(700 + M, M, K, N, dtype, 128)
    packed = pack_on_gpu(w, ws)
    bias_bits = None
    bias = None
    if with_bias:
        rng = np.random.default_rng(M)
        bias_bits = numerics.f64_to_half_bits_rne(rng.standard_normal(N), dtype)
        bias = bits_to_device(bias_bits, dtype)
    y = run(w, ws, packed, ws.x_bits[M], path="mfma", bias=bias)
    y2 = run(w, ws, packed, ws.x_bits[M], path="mfma", bias=bias)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    got = y_to_f64(y, dtype)
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[M], bias_bits=bias_bits)) <= TOL


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_bias(w, path):
    ws = synth.make_custom(60, 8, 1024, 272, "bf16", 128)
    rng = np.random.default_rng(60)
    bias_bits = numerics.f64_to_half_bits_rne(rng.standard_normal(272), "bf16")
    packed = pack_on_gpu(w, ws)
    got = y_to_f64(run(w, ws, packed, ws.x_bits[8], path=path, bias=bits_to_device(bias_bits, "bf16")), "bf16")
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[8], bias_bits=bias_bits)) <= TOL


@pytest.mark.parametrize("M", [1, 8, 16, 512])
def test_deterministic_and_in_bounds(w, M):
    ws = synth.make_custom(70 + M, M, 2048, 1040, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[M], "bf16")
    pad = 4096
    outs = []
    for _ in range(2):
        buf = torch.full((M * 1040 + 2 * pad,), -7.0, dtype=torch.bfloat16, device=DEV)
        y = buf[pad:pad + M * 1040].view(M, 1040)
        w.w4a16_gemm(x, packed, 1040, 128, y=y)
        torch.cuda.synchronize()
        b = buf.cpu()
        assert torch.all(b[:pad] == -7.0) and torch.all(b[-pad:] == -7.0), "write outside y"
        outs.append(device_to_bits(y))
    assert np.array_equal(outs[0], outs[1])


def test_side_stream(w):
    ws = synth.make_custom(80, 64, 1024, 512, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[64], "bf16")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y1 = w.w4a16_gemm(x[:4].contiguous(), packed, 512, 128, stream=s)
        y2 = w.w4a16_gemm(x, packed, 512, 128, stream=s)
    s.synchronize()
    assert ogemm.max_rel_error(y_to_f64(y2, "bf16"), oracle_y(ws, ws.x_bits[64])) <= TOL
    assert ogemm.max_rel_error(y_to_f64(y1, "bf16"), oracle_y(ws, ws.x_bits[64][:4])) <= TOL


def test_edge_shapes(w):
    # one row block and one column block; M = 0 is a no-op
    ws = synth.make_custom(90, 3, 128, 16, "fp16", 128)
    packed = pack_on_gpu(w, ws)
    for path in ("gemv", "mfma"):
        got = y_to_f64(run(w, ws, packed, ws.x_bits[3], path=path), "fp16")
        assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[3])) <= TOL
    x0 = torch.empty((0, 128), dtype=torch.float16, device=DEV)
    y0 = w.w4a16_gemm(x0, packed, 16, 128)
    assert y0.shape == (0, 16)


def test_per_channel_and_wide_groups(w):
    for G in (-1, 256):
        ws = synth.make_custom(95, 20, 1024, 64, "bf16", G)
        packed = pack_on_gpu(w, ws)
        for path, M in (("gemv", 5), ("mfma", 20)):
            xb = ws.x_bits[20][:M]
            got = y_to_f64(run(w, ws, packed, xb, path=path), "bf16")
            assert ogemm.max_rel_error(got, oracle_y(ws, xb)) <= TOL


def test_gemm_rejects_bad_calls(w):
    ws = synth.make_custom(99, 4, 256, 32, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[4], "bf16")
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_gemm(x, packed[:100], 32, 128)
    assert e.value.status == "W4A16_ERR_BUFFER_SIZE"
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_gemm_ex(x, packed, 32, 128, path="gemv", gemv_max_m=17)
    assert e.value.status == "W4A16_ERR_PATH"
    xbig = torch.zeros((17, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_gemm_ex(xbig, packed, 32, 128, path="gemv")
    assert e.value.status == "W4A16_ERR_PATH"
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_gemm(x, packed, 32, 96)
    assert e.value.status == "W4A16_ERR_GROUP"


@pytest.mark.parametrize("M,K,N,path,G", [
    (8, 2048, 20480, "gemv", 128),     # M <= 8: the GEMV at every size
    (9, 2048, 20480, "mfma", 128),     # 20 MiB of codes: the MFMA GEMM from M = 9
    (12, 2048, 13312, "gemv", 128),    # 832 column blocks, at most 7 half blocks per compute unit:
    (16, 2048, 13312, "gemv", 128),    # the balanced matrix-core GEMV through M = 16
    (13, 2048, 16400, "mfma", 128),    # 15.6 MiB, 9 half blocks per compute unit: the MFMA GEMM from M = 13
    (15, 2048, 3072, "gemv", 128),     # 3 MiB: the GEMV through M = 15
    (16, 2048, 3072, "mfma", 128),     # M >= 16: the MFMA GEMM at every size
    (9, 2048, 3072, "mfma", 64),       # groups of 64 rows keep the stated M <= 8
    (15, 6656, 2048, "gemv", 128),     # N <= 2048: the GEMV (K split) through M = 15
    (16, 6656, 2048, "mfma", 128),
])
def test_default_dispatch_follows_weight_size(w, M, K, N, path, G):
    ws = synth.make_custom(130 + M, M, K, N, "bf16", G)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[M], "bf16")
    auto = device_to_bits(w.w4a16_gemm(x, packed, N, G))
    forced = device_to_bits(w.w4a16_gemm_ex(x, packed, N, G, path=path))
    torch.cuda.synchronize()
    assert np.array_equal(auto, forced), (M, K, N, path, G)
    if N == 3072:
        ref = oracle_y(ws, ws.x_bits[M])
        assert ogemm.max_rel_error(numerics.half_bits_to_f64(auto, "bf16"), ref) <= TOL


def test_split_k_workspace_is_reused_and_left_zero(w):
    # a skinny shape whose MFMA GEMM splits K over workgroups: three calls on one
    # zeroed workspace must agree bit for bit (the tile counters are reset each call),
    # then another split shape on the same workspace
    ws = synth.make_custom(110, 16, 6656, 2048, "bf16", 128)
    need = w.w4a16_workspace_bytes(16, 6656, 2048, 128)
    assert need > 0
    work = torch.zeros(need + 4096, dtype=torch.uint8, device=DEV)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[16], "bf16")
    outs = []
    for _ in range(3):
        y = w.w4a16_gemm_ex(x, packed, 2048, 128, workspace=work, path="mfma")
        torch.cuda.synchronize()
        outs.append(device_to_bits(y))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    ref = oracle_y(ws, ws.x_bits[16])
    assert ogemm.max_rel_error(numerics.half_bits_to_f64(outs[0], "bf16"), ref) <= TOL
    ws2 = synth.make_custom(111, 40, 2560, 96, "bf16", 128)
    assert w.w4a16_workspace_bytes(40, 2560, 96, 128) > 0
    packed2 = pack_on_gpu(w, ws2)
    y2 = w.w4a16_gemm_ex(bits_to_device(ws2.x_bits[40], "bf16"), packed2, 96, 128, workspace=work, path="mfma")
    torch.cuda.synchronize()
    assert ogemm.max_rel_error(y_to_f64(y2, "bf16"), oracle_y(ws2, ws2.x_bits[40])) <= TOL
    # the counter part of the workspace (one fixed 512-byte region) is zero again
    assert int(work[:512].count_nonzero()) == 0


def test_split_k_workspace_shared_across_growing_shapes(w):
    # one zeroed workspace serves split-K calls of different shapes in any order: a
    # call with 32 output tiles (K split 8 ways) leaves fp32 partials behind its
    # counters, and a later call with 96 tiles (split 3 ways) and the W4A8 GEMM on
    # that shape must still find all of their counters at zero. Each result agrees
    # bit for bit with the same call on a fresh workspace.
    shapes = [(16, 6656, 2048), (16, 2048, 6144)]
    needs = [w.w4a16_workspace_bytes(M, K, N, 128) for M, K, N in shapes]
    assert all(n > 0 for n in needs)
    assert w.w4a8_workspace_bytes(16, 2048, 6144, 128) == needs[1]
    cases = []
    for seed, (M, K, N) in zip((120, 121), shapes):
        ws = synth.make_custom(seed, M, K, N, "bf16", 128)
        cases.append((ws, pack_on_gpu(w, ws), bits_to_device(ws.x_bits[M], "bf16")))

    def w4a16(i, work):
        ws, packed, x = cases[i]
        return device_to_bits(w.w4a16_gemm_ex(x, packed, ws.N, 128, workspace=work, path="mfma"))

    def w4a8(i, work):
        ws, packed, x = cases[i]
        M, K, N = shapes[i]
        act = w.w4a8_quantize(x)
        return device_to_bits(w.w4a8_gemm(act, packed, M, K, N, 128, torch.bfloat16, workspace=work))

    fresh = lambda n: torch.zeros(n, dtype=torch.uint8, device=DEV)
    want = [w4a16(0, fresh(needs[0])), w4a16(1, fresh(needs[1])), w4a8(1, fresh(needs[1]))]
    torch.cuda.synchronize()
    for i in (0, 1):
        ws = cases[i][0]
        got = numerics.half_bits_to_f64(want[i], "bf16")
        assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[shapes[i][0]])) <= TOL
    shared = fresh(max(needs))
    order = [("w4a16", 0), ("w4a16", 1), ("w4a8", 1), ("w4a16", 0), ("w4a8", 1), ("w4a16", 1)]
    for kind, i in order:
        got = w4a16(i, shared) if kind == "w4a16" else w4a8(i, shared)
        torch.cuda.synchronize()
        assert np.array_equal(got, want[i] if kind == "w4a16" else want[2]), (kind, shapes[i])
    assert int(shared[:512].count_nonzero()) == 0


def test_split_k_default_workspace_per_stream(w):
    # split-K calls on two streams with no workspace passed: the binding gives each
    # stream its own zeroed workspace, so calls queued on both at once do not meet in
    # each other's tile counters; every result matches the one-stream result bit for bit
    ws = synth.make_custom(113, 16, 6656, 2048, "bf16", 128)
    assert w.w4a16_workspace_bytes(16, 6656, 2048, 128) > 0
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[16], "bf16")
    want = device_to_bits(w.w4a16_gemm_ex(x, packed, 2048, 128, path="mfma"))
    torch.cuda.synchronize()
    assert ogemm.max_rel_error(numerics.half_bits_to_f64(want, "bf16"), oracle_y(ws, ws.x_bits[16])) <= TOL
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    ys = []
    for i in range(8):
        s = streams[i % 2]
        with torch.cuda.stream(s):
            ys.append(w.w4a16_gemm_ex(x, packed, 2048, 128, path="mfma", stream=s))
    torch.cuda.synchronize()
    for y in ys:
        assert np.array_equal(device_to_bits(y), want)
    keys = {k for k in w._workspaces if k[0] == torch.device(DEV).index}
    assert {(torch.device(DEV).index, s.cuda_stream) for s in streams} <= keys


def test_split_k_rejects_small_workspace(w):
    ws = synth.make_custom(112, 16, 6656, 2048, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[16], "bf16")
    small = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_gemm_ex(x, packed, 2048, 128, workspace=small, path="mfma")
    assert e.value.status == "W4A16_ERR_BUFFER_SIZE"


@pytest.mark.parametrize("K", [8320, 9216])
@pytest.mark.parametrize("M", [1, 5, 16])
def test_gemv_long_k(w, K, M):
    # more than 64 row blocks: each wave takes several runs of 4 row blocks, the next
    # run's loads in flight during the current one (65 row blocks: 9 waves of 8, the
    # last with one valid block); M = 16 does not fit in LDS and reads x directly
    ws = synth.make_custom(700 + M + K // 128, M, K, 48, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    got = y_to_f64(run(w, ws, packed, ws.x_bits[M], path="gemv"), "bf16")
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[M])) <= TOL


@pytest.mark.parametrize("M,K,N,dtype", [(8, 6656, 2048, "bf16"), (12, 6656, 2048, "fp16"),
                                         (16, 6656, 2048, "bf16"), (6, 8192, 1000, "bf16"),
                                         (9, 6656, 1280, "fp16"), (1, 6656, 2048, "bf16"),
                                         (8, 2048, 2048, "bf16")])
def test_gemv_k_split_over_workgroups(w, M, K, N, dtype):
    # narrow outputs (at most 128 column blocks) with K >= 6144 split each block's K
    # range over 2-4 workgroups from M = 9 when the workspace holds their partials
    # (N = 2048: 2 ways, N = 1280: 3); M = 1 runs the balanced GEMV, M = 2 .. 8 the
    # balanced matrix-core GEMV (M = 8 and M = 6 with N = 1000 here), K = 2048 keeps one
    # workgroup per block, and none of those touch the workspace: parity with the
    # oracle, the same result on a second call, the counters left at zero, nothing
    # written outside y (N = 1000: a ragged last block); without a workspace one
    # workgroup per block gives a result within the same tolerance
    print(f"gemv K split over workgroups M={M} K={K} N={N} {dtype}", flush=True)
    ws = synth.make_custom(150 + M, M, K, N, dtype, 128)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[M], dtype)
    ref = oracle_y(ws, ws.x_bits[M])
    need = w.w4a16_workspace_bytes(M, K, N, 128)
    assert need > 0
    work = torch.zeros(need, dtype=torch.uint8, device=DEV)
    pad = 4096
    outs = []
    for _ in range(2):
        buf = torch.full((M * N + 2 * pad,), -7.0, dtype=TORCH_DTYPE[dtype], device=DEV)
        y = buf[pad:pad + M * N].view(M, N)
        w.w4a16_gemm_ex(x, packed, N, 128, y=y, workspace=work, path="gemv")
        torch.cuda.synchronize()
        b = buf.cpu()
        assert torch.all(b[:pad] == -7.0) and torch.all(b[-pad:] == -7.0), "write outside y"
        outs.append(device_to_bits(y))
    assert np.array_equal(outs[0], outs[1])
    assert int(work[:512].count_nonzero()) == 0
    # the partials region shows whether the split ran: written by the split cases,
    # untouched by the balanced GEMVs (M <= 8) and by K = 2048
    splits = M > 8 and K >= 6144
    assert (int(work[512:].count_nonzero()) > 0) == splits, (M, K, N)
    assert ogemm.max_rel_error(numerics.half_bits_to_f64(outs[0], dtype), ref) <= TOL
    none = torch.empty(0, dtype=torch.uint8, device=DEV)
    y1 = w.w4a16_gemm_ex(x, packed, N, 128, workspace=none, path="gemv")
    torch.cuda.synchronize()
    assert ogemm.max_rel_error(y_to_f64(y1, dtype), ref) <= TOL


def test_gemv_needs_no_workspace(w):
    # a NULL workspace (an empty buffer; None would get the binding's default) on a
    # shape whose GEMV would split K over workgroups given one: one workgroup per block
    ws = synth.make_custom(140, 12, 6656, 2048, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[12], "bf16")
    none = torch.empty(0, dtype=torch.uint8, device=DEV)
    y = w.w4a16_gemm_ex(x, packed, 2048, 128, workspace=none, path="gemv")
    torch.cuda.synchronize()
    assert ogemm.max_rel_error(y_to_f64(y, "bf16"), oracle_y(ws, ws.x_bits[12])) <= TOL


@pytest.mark.parametrize("K,M,N,dtype", [(2048, 1, 13296, "bf16"), (2048, 9, 13296, "bf16"),
                                         (2048, 3, 13296, "fp16"), (512, 2, 13296, "bf16"),
                                         (1024, 3, 13296, "bf16"), (1024, 4, 16400, "bf16"),
                                         (1024, 8, 16400, "fp16")])
def test_gemv_several_column_blocks_per_workgroup(w, K, M, N, dtype):
    # the 16-column GEMV: N = 13296 (831 column blocks) runs 2 blocks per workgroup at
    # every M it takes (M = 4 .. 8 there go to the balanced matrix-core GEMV), N = 16400
    # (1025 blocks, beyond that kernel's 8 units per lane) from M = 4: the last
    # workgroup has a block past N, which repeats the last block and must store
    # nothing. K = 512 has one wave per block (no K split), K = 1024 two.
    print(f"gemv 2 blocks per workgroup K={K} M={M} N={N} {dtype}", flush=True)
    ws = synth.make_custom(1000 + K // 128 + M, M, K, N, dtype, 128)
    packed = pack_on_gpu(w, ws)
    x = bits_to_device(ws.x_bits[M], dtype)
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), -7.0, dtype=TORCH_DTYPE[dtype], device=DEV)
    y = buf[pad:pad + M * N].view(M, N)
    w.w4a16_gemm_ex(x, packed, N, 128, y=y, path="gemv")
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:pad] == -7.0) and torch.all(b[-pad:] == -7.0), "write outside y"
    assert ogemm.max_rel_error(y_to_f64(y, dtype), oracle_y(ws, ws.x_bits[M])) <= TOL


@pytest.mark.parametrize("M", [300, 512])
def test_gemm_wide_n(w, M):
    # LM-head width (8192 column blocks, 512 column tiles of 256) with a short K;
    # M = 300 leaves a ragged third row tile; the whole output
    ws = synth.make_custom(800 + M, M, 256, 131072, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    got = y_to_f64(run(w, ws, packed, ws.x_bits[M], path="mfma"), "bf16")
    err, _ = whole_output_error(got, lambda cols: oracle_y(ws, ws.x_bits[M], cols))
    assert err <= TOL


@pytest.mark.parametrize("M,N,dtype", [(500, 13264, "bf16"), (500, 13264, "fp16"), (250, 13264, "bf16"),
                                       (3000, 2608, "bf16"), (20, 131072, "bf16"), (480, 3080, "bf16"),
                                       (480, 3080, "fp16"), (1000, 2600, "bf16"), (1000, 2600, "fp16"),
                                       (48, 65528, "bf16")])
def test_gemm_tile_shapes(w, M, N, dtype):
    # 256-column tiles run as 8 waves of 2 column blocks: N = 13264 (829 blocks) leaves
    # a last tile whose last wave lies wholly past N, M = 500 a ragged last row tile
    # (128-row tiles); M = 48, N = 65528 takes 64 x 256 tiles (a ragged row tile, a
    # half last block); M = 20 is the shortest 8-wave tile (32 rows: one activation copy
    # per wave). 128 x 128 tiles as 8 waves of one block: M = 250 and M = 3000 (N = 2608,
    # the last tile 3 blocks wide), M = 1000, N = 2600 (ragged rows, a half last block).
    # 64 x 128 tiles as 8 waves of one block: M = 480, N = 3080 (ragged rows, a half
    # last block). The whole output, wide N in column chunks.
    ws = synth.make_custom(900 + M % 97, M, 256, N, dtype, 128)
    packed = pack_on_gpu(w, ws)
    got = y_to_f64(run(w, ws, packed, ws.x_bits[M], path="mfma"), dtype)
    err, _ = whole_output_error(got, lambda cols: oracle_y(ws, ws.x_bits[M], cols))
    assert err <= TOL


@pytest.mark.parametrize("K,N,dtype,G,bias", [
    (2048, 13312, "bf16", 128, False),   # 1664 half blocks on 256 workgroups: 6 or 7 each, 1 row block per group
    (6656, 2048, "bf16", 128, True),     # one half block per workgroup, 4 row blocks per group, 52 of 64 groups busy
    (128, 8, "fp16", 128, False),        # one workgroup, one half block, 4 of 64 groups busy
    (256, 24, "bf16", 128, True),        # a last half block (N % 16 == 8), 3 workgroups
    (16384, 2056, "bf16", 128, False),   # 8 row blocks per group would be needed: the 16-column GEMV runs
    (4096, 4104, "fp16", 256, True),     # 2 row blocks per group, 3 half blocks per workgroup, groups of 256
    (2176, 520, "fp16", 128, True),      # 17 row blocks in runs of 2: the last group has one
    (6784, 1032, "bf16", 128, False),    # 53 row blocks in runs of 4: the last group has one; N % 16 == 8
    (8192, 2048, "bf16", 128, True),     # 64 row blocks: every group busy with 4
    (1536, 1040, "bf16", -1, False),     # one group of all K rows
    # shares dealt over the XCDs (grids that are a multiple of 8; 65, 129 and 130 above are not)
    (2048, 1024, "bf16", 128, True),     # 128 workgroups, one half block each
    (3072, 512, "fp16", 128, False),     # 64 workgroups, 2 row blocks per group
    (2048, 2064, "bf16", 128, True),     # 258 half blocks on 256 workgroups: two take two
    (2048, 10240, "fp16", 128, False),   # 5 half blocks per workgroup
    (1024, 12288, "bf16", 128, True),    # 6 half blocks per workgroup
    (1024, 40000, "bf16", 128, False),   # 20 half blocks per workgroup: beyond the balanced GEMV, the
                                         # 16-column GEMV runs
])
def test_gemv_m1_balanced_half_blocks(w, K, N, dtype, G, bias):
    print(f"gemv M=1 K={K} N={N} {dtype} G={G} bias={bias}", flush=True)
    ws = synth.make_custom(1700 + K % 997 + N % 89, 1, K, N, dtype, G)
    packed = pack_on_gpu(w, ws)
    bias_bits = None
    bt = None
    if bias:
        rng = np.random.default_rng(N)
        bias_bits = synth.f32_to_half_bits(rng.standard_normal(N, dtype=np.float32), dtype)
        bt = bits_to_device(bias_bits, dtype)
    x = bits_to_device(ws.x_bits[1], dtype)
    pad = 256
    buf = torch.full((2 * pad + N,), -7.0, dtype=TORCH_DTYPE[dtype], device=DEV)
    y = buf[pad:pad + N].view(1, N)
    w.w4a16_gemm(x, packed, N, G, bias=bt, y=y)
    y2 = w.w4a16_gemm(x, packed, N, G, bias=bt)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:pad] == -7.0) and torch.all(b[-pad:] == -7.0), "write outside y"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not run-to-run deterministic"
    err = ogemm.max_rel_error(y_to_f64(y, dtype), oracle_y(ws, ws.x_bits[1], bias_bits=bias_bits))
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("M,K,N,dtype,G,bias", [
    (2, 6656, 2048, "bf16", 128, True),    # 128 column blocks: M = 2 takes it; 26 units, 4 per wave
    (8, 6656, 2048, "fp16", 128, False),   # the down_proj decode shape at M = 8
    (5, 2048, 13312, "bf16", 128, True),   # 6 or 7 half blocks per workgroup, one unit each per wave
    (4, 2048, 3072, "fp16", 128, False),   # 1 or 2 half blocks per workgroup
    (7, 1152, 272, "bf16", 128, False),    # 9 row blocks: the last unit lacks its second row block
    (6, 1408, 264, "bf16", 128, True),     # N % 16 == 8 (a last lower half block), 11 row blocks
    (3, 1536, 1040, "bf16", -1, False),    # 65 column blocks: M = 3 takes it; one group of all K rows
    (8, 16384, 520, "bf16", 256, True),    # 64 units per half block: 8 per wave; G = 256
    (4, 128, 8, "fp16", 128, False),       # one workgroup, one unit with one row block
    (8, 2048, 4104, "bf16", 128, False),   # 513 half blocks: workgroups of 2 and 3
    (12, 2048, 13312, "bf16", 128, True),  # two row groups (8 + 4 rows) on a wide output
    (16, 1024, 8200, "fp16", 128, False),  # two full row groups; 1025 half blocks, 4 or 5 per workgroup
    (9, 2304, 8192, "bf16", 128, True),    # a second group of one row; 9 units per half block
])
def test_gemv_small_batch_matrix_cores(w, M, K, N, dtype, G, bias):
    # the balanced matrix-core GEMV for 2 <= M <= 16: the whole output against the
    # oracle, bias, run-to-run identical results, nothing written outside y
    print(f"gemv small batch M={M} K={K} N={N} {dtype} G={G} bias={bias}", flush=True)
    ws = synth.make_custom(1900 + M + K % 991 + N % 83, M, K, N, dtype, G)
    packed = pack_on_gpu(w, ws)
    bias_bits = None
    bt = None
    if bias:
        rng = np.random.default_rng(N + M)
        bias_bits = synth.f32_to_half_bits(rng.standard_normal(N, dtype=np.float32), dtype)
        bt = bits_to_device(bias_bits, dtype)
    x = bits_to_device(ws.x_bits[M], dtype)
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), -7.0, dtype=TORCH_DTYPE[dtype], device=DEV)
    y = buf[pad:pad + M * N].view(M, N)
    w.w4a16_gemm_ex(x, packed, N, G, bias=bt, y=y, path="gemv")
    y2 = w.w4a16_gemm(x, packed, N, G, bias=bt)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:pad] == -7.0) and torch.all(b[-pad:] == -7.0), "write outside y"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not run-to-run deterministic"
    err = ogemm.max_rel_error(y_to_f64(y, dtype), oracle_y(ws, ws.x_bits[M], bias_bits=bias_bits))
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL
