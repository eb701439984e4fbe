"""w4a16_gemm_noalloc, the GEMM entry point that allocates nothing: its K-split
partials live in the library's own per-GPU array. Each call must return exactly
what w4a16_gemm returns with a caller workspace (same plan, same kernels), and
stay within the oracle's tolerance."""

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from gpu_util import DEV, bits_to_device, oracle_y, weights_to_device, y_to_f64

pytestmark = pytest.mark.gpu
TOL = ogemm.TOLERANCE

# (seed, M, K, N): MFMA GEMM splitting K over 8 workgroups, GEMV splitting K over 2
# workgroups per column block, then a GEMV that uses no scratch; each smaller than
# the one before.
SEQUENCE = [(1601, 16, 6656, 2048), (1602, 8, 6656, 2048), (1603, 1, 2048, 512)]


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def _case(w, seed, M, K, N):
    ws = synth.make_custom(seed, M, K, N, "bf16", 128)
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, 128)
    x = bits_to_device(ws.x_bits[M], "bf16")
    need = w.w4a16_workspace_bytes(M, K, N, 128)
    workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    y_ref = w.w4a16_gemm(x, packed, N, 128, workspace=workspace)
    torch.cuda.synchronize()
    return ws, packed, x, y_ref


@pytest.mark.parametrize("rounds", [2])
def test_noalloc_matches_workspace_gemm(w, rounds):
    cases = [(_case(w, *c), c) for c in SEQUENCE]
    for r in range(rounds):
        for (ws, packed, x, y_ref), (seed, M, K, N) in cases:
            print(f"noalloc round {r} M={M} K={K} N={N}", flush=True)
            y = torch.full((M, N), -3.0, dtype=torch.bfloat16, device=DEV)
            torch.cuda.synchronize()
            before = torch.cuda.memory_allocated()
            w.w4a16_gemm_noalloc(x, packed, N, 128, y=y)
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated() == before
            # the same kernels and plan as the workspace call: bit for bit
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (r, M, K, N)
            err = ogemm.max_rel_error(y_to_f64(y, "bf16"), oracle_y(ws, ws.x_bits[M]))
            print(f"  max rel err {err:.3e}", flush=True)
            assert err <= TOL


def test_noalloc_bias_and_fp16(w):
    ws = synth.make_custom(1611, 12, 6656, 1024, "fp16", 128)
    rng = np.random.default_rng(3)
    bias_bits = synth.f32_to_half_bits(rng.standard_normal(1024, dtype=np.float32), "fp16")
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, 128)
    x = bits_to_device(ws.x_bits[12], "fp16")
    bias = bits_to_device(bias_bits, "fp16")
    y = w.w4a16_gemm_noalloc(x, packed, 1024, 128, bias=bias)
    ws_buf = torch.zeros(max(w.w4a16_workspace_bytes(12, 6656, 1024, 128), 256), dtype=torch.uint8, device=DEV)
    y_ref = w.w4a16_gemm(x, packed, 1024, 128, bias=bias, workspace=ws_buf)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    err = ogemm.max_rel_error(y_to_f64(y, "fp16"), oracle_y(ws, ws.x_bits[12], bias_bits=bias_bits))
    assert err <= TOL


def test_noalloc_rejects_a_split_beyond_its_array(w):
    # M = 33, K = 16384, N = 512: the MFMA GEMM's split partials need more than the
    # array holds; the call is refused on the host, nothing is launched
    M, K, N = 33, 16384, 512
    assert w.w4a16_workspace_bytes(M, K, N, 128) > w.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    packed = torch.zeros(w.w4a16_packed_bytes(K, N, 128), dtype=torch.uint8, device=DEV)
    y = torch.full((M, N), 5.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_gemm_noalloc(x, packed, N, 128, y=y)
    assert e.value.status == "W4A16_ERR_BUFFER_SIZE"
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)
