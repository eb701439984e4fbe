"""The C-ABI library on the host: it loads without a GPU, exports every entry point
the header declares, and rejects invalid arguments before touching a device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a(?:16|8)_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "w4a16_embedding", "w4a16_gemm", "w4a16_gemm_ex", "w4a16_gemm_noalloc", "w4a16_layout_version",
        "w4a16_packed_bytes",
        "w4a16_packed_header", "w4a16_parse_packed_header", "w4a16_repack", "w4a16_repack_columns",
        "w4a16_repack_gptq", "w4a16_repack_gptq_columns", "w4a16_status_str", "w4a16_workspace_bytes",
        "w4a8_activation_bytes", "w4a8_gemm", "w4a8_quantize", "w4a8_workspace_bytes"])


def test_library_exports_every_declared_symbol(w):
    for name in declared_functions():
        assert hasattr(w.lib, name), name
    # and the binding mirrors each name
    for name in declared_functions():
        assert callable(getattr(w, name)), name


def measure_functions():
    text = open(os.path.join(ROOT, "include", "w4a16_measure.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z_0-9]+)\s*\(", text)))


def test_measure_header_entry_points_are_exported_and_bound(w):
    import subprocess
    from w4a16_int4_weight_amd.build import LIB_PATH
    assert measure_functions() == ["w4a16_clock_stamp", "w4a16_stream_copy", "w4a16_stream_read",
                                   "w4a16_stream_sink_bytes", "w4a16_wall_clock_hz"]
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in measure_functions():
        assert name in exported and callable(getattr(w, name)), name


def test_stream_validation_before_any_device_call(w):
    assert w.w4a16_stream_sink_bytes(0) == 0
    assert w.w4a16_stream_sink_bytes(24) == 0
    assert w.w4a16_stream_sink_bytes(16) == 16                       # one chunk: one workgroup
    assert w.w4a16_stream_sink_bytes(32768) == 512 * 16               # 512, 768 or 1024 shares up to 64 MiB
    assert w.w4a16_stream_sink_bytes(14_194_688) == 1024 * 16         # 866 16-KiB pieces: rounded up to 1024
    assert w.w4a16_stream_sink_bytes(10 << 20) == 768 * 16            # 640: rounded up to 768
    assert w.w4a16_stream_sink_bytes(7_099_392) == 512 * 16
    assert w.w4a16_stream_sink_bytes(64 << 20) == 1024 * 16
    assert w.w4a16_stream_sink_bytes((64 << 20) + 16) == ((64 << 20) // 16 + 1 + 2047) // 2048 * 16
    lib = w.lib
    assert lib.w4a16_stream_read(P(256), 24, P(512), 16, None) == 2
    assert lib.w4a16_stream_read(None, 32, P(512), 16, None) == 1
    assert lib.w4a16_stream_read(P(256), 32, None, 16, None) == 1
    assert lib.w4a16_stream_read(P(260), 32, P(512), 16, None) == 5
    assert lib.w4a16_stream_read(P(256), 32768 + 16, P(512), 16, None) == 6
    assert lib.w4a16_stream_read(P(256), 32768, P(512), 512 * 16 - 1, None) == 6
    assert lib.w4a16_stream_read(None, 0, None, 0, None) == 0
    assert lib.w4a16_stream_copy(P(256), P(512), 40, None) == 2
    assert lib.w4a16_stream_copy(P(256), None, 32, None) == 1
    assert lib.w4a16_stream_copy(P(256), P(520), 32, None) == 5
    assert lib.w4a16_stream_copy(None, None, 0, None) == 0
    assert lib.w4a16_clock_stamp(None, None) == 1
    assert lib.w4a16_clock_stamp(P(260), None) == 5
    assert lib.w4a16_wall_clock_hz(None) == 1


def test_exports_are_c_symbols():
    # no C++ mangling on the entry points
    import subprocess
    from w4a16_int4_weight_amd.build import LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name


def test_layout_version_and_sizes(w):
    from oracle import tile_layout
    assert w.w4a16_layout_version() == tile_layout.LAYOUT_VERSION
    for K, N, G in [(512, 512, 128), (2048, 13312, 128), (6656, 2048, 128), (2048, 131072, 128),
                    (1024, 48, 256), (1024, 48, -1), (256, 24, 128), (2048, 13288, 128), (384, 40, 64),
                    (384, 40, 32), (6656, 2048, 32)]:
        assert w.w4a16_packed_bytes(K, N, G) == tile_layout.packed_bytes(K, N, G)
    for K, N, G in [(100, 16, 128), (256, 20, 128), (256, 16, 96), (384, 16, 256), (0, 16, 128), (128, 0, 128)]:
        assert w.w4a16_packed_bytes(K, N, G) == 0
    # K split over workgroups only when the output has too few tiles for the GPU
    assert w.w4a16_workspace_bytes(512, 2048, 131072, 128) == 0
    assert w.w4a16_workspace_bytes(512, 2048, 13312, 128) == 0
    ws = w.w4a16_workspace_bytes(16, 6656, 2048, 128)
    assert ws > 16 * 2048 * 4 and ws % 4 == 0
    # a split plan's workspace: 128 tile counters (512 bytes) whatever its tile count,
    # then fp32 partial tiles of 16 x 64 per tile and split (32 tiles x 8 splits here;
    # 96 tiles x 3 splits at N = 6144, K = 2048), so no shape's partials overlap
    # another shape's counters
    assert ws == 512 + 8 * 32 * 16 * 64 * 4
    assert w.w4a16_workspace_bytes(16, 2048, 6144, 128) == 512 + 3 * 96 * 16 * 64 * 4
    assert w.w4a16_workspace_bytes(16, 6656, 2048, 96) == 0          # invalid group size
    # sized for the MFMA GEMM, which any M may be sent to; the GEMV needs none
    assert w.w4a16_workspace_bytes(1, 2048, 131072, 128) == 0
    assert w.w4a16_workspace_bytes(0, 6656, 2048, 128) == 0


def test_status_strings(w):
    for code in range(11):
        s = w.w4a16_status_str(code)
        assert s and s != "unknown status"
    assert w.w4a16_status_str(42) == "unknown status"


P = ctypes.c_void_p


def gemm(w, x=P(256), packed=P(512), pbytes=1 << 40, dtype=1, y=P(1024), M=4, K=512, N=512, G=128,
         bias=None, ws=None, wsb=0, stream=None, path=None, gmax=-1):
    args = (x, packed, pbytes, dtype, y, M, K, N, G, bias, ws, wsb, stream)
    if path is None:
        return w.lib.w4a16_gemm(*args)
    return w.lib.w4a16_gemm_ex(*args, path, gmax)


def test_gemm_validation_before_any_device_call(w):
    # each invalid call returns its status; none reaches the device check (7)
    assert gemm(w, M=-1) == 2
    assert gemm(w, K=500) == 2
    assert gemm(w, N=20) == 2
    assert gemm(w, K=0) == 2
    assert gemm(w, K=(1 << 20) + 128) == 2
    assert gemm(w, N=(1 << 28) + 16) == 2
    assert gemm(w, K=1 << 20, N=1 << 18) == 2
    assert gemm(w, M=1 << 13, K=1 << 20) == 2
    assert gemm(w, G=96) == 3
    assert gemm(w, G=384) == 3
    assert gemm(w, dtype=2) == 4
    assert gemm(w, x=None) == 1
    assert gemm(w, packed=None) == 1
    assert gemm(w, y=None) == 1
    assert gemm(w, x=P(258)) == 5
    assert gemm(w, packed=P(520)) == 5
    assert gemm(w, y=P(1032)) == 5
    assert gemm(w, bias=P(1025)) == 5
    assert gemm(w, pbytes=512 * 512 // 2) == 6
    assert gemm(w, path=3) == 9
    assert gemm(w, path=1, M=17) == 9
    assert gemm(w, path=0, gmax=17) == 9
    # a shape whose MFMA GEMM splits K needs the workspace
    assert gemm(w, M=16, K=6656, N=2048, path=2) == 1
    assert gemm(w, M=16, K=6656, N=2048, path=2, ws=P(4096), wsb=64) == 6
    assert gemm(w, M=16, K=6656, N=2048, path=2, ws=P(4100), wsb=1 << 30) == 5
    assert gemm(w, M=16, K=6656, N=2048, path=1) == 7                   # GEMV needs none
    assert gemm(w, M=1, K=6656, N=2048) == 7
    # M = 0 is a valid no-op, even with NULL buffers
    assert gemm(w, M=0, x=None, y=None, packed=None) == 0
    # a fully valid call on this GPU-less host stops at the device check
    assert gemm(w) == 7


def test_gemm_noalloc_validation_before_any_device_call(w):
    def noalloc(x=P(256), packed=P(512), pbytes=1 << 40, dtype=1, y=P(1024), M=4, K=512, N=512, G=128, bias=None):
        return w.lib.w4a16_gemm_noalloc(x, packed, pbytes, dtype, y, M, K, N, G, bias, None)
    assert noalloc(M=-1) == 2
    assert noalloc(K=500) == 2
    assert noalloc(G=96) == 3
    assert noalloc(dtype=2) == 4
    assert noalloc(x=None) == 1
    assert noalloc(y=P(1032)) == 5
    assert noalloc(pbytes=512 * 512 // 2) == 6
    assert noalloc(M=0, x=None, y=None, packed=None) == 0
    # a split plan whose partials exceed the library's array: rejected before the device
    big = dict(M=33, K=16384, N=512)
    assert w.w4a16_workspace_bytes(33, 16384, 512, 128) > w.NOALLOC_SCRATCH_BYTES
    assert noalloc(**big) == 6
    # split plans within the array, and plans with no split, reach the device check
    assert 0 < w.w4a16_workspace_bytes(16, 6656, 2048, 128) <= w.NOALLOC_SCRATCH_BYTES
    assert noalloc(M=16, K=6656, N=2048) == 7
    assert noalloc(M=8, K=6656, N=2048) == 7
    assert noalloc() == 7
    # every M <= 32 fits the array (the split plans' partials stay below it)
    for M in (1, 8, 16, 17, 32):
        for K in (2048, 6656, 65536, 1 << 20):
            for N in (16, 512, 2048, 8192):
                assert w.w4a16_workspace_bytes(M, K, N, 128) <= w.NOALLOC_SCRATCH_BYTES, (M, K, N)


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "w4a16.h")).read()
    m = re.search(r"#define W4A16_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    import w4a16_int4_weight_amd as mod
    assert m and int(m.group(1)) << int(m.group(2)) == mod.NOALLOC_SCRATCH_BYTES


def test_repack_validation_before_any_device_call(w):
    def repack(qw=P(256), qz=P(512), sc=P(768), dtype=1, K=512, N=512, G=128, packed=P(1024), pbytes=1 << 40):
        return w.lib.w4a16_repack(qw, qz, sc, dtype, K, N, G, packed, pbytes, None)
    assert repack(K=100) == 2
    assert repack(N=12) == 2
    assert repack(G=96) == 3
    assert repack(dtype=-1) == 4
    assert repack(qw=None) == 1
    assert repack(qz=None) == 1
    assert repack(sc=None) == 1
    assert repack(packed=None) == 1
    assert repack(qw=P(258)) == 5
    assert repack(sc=P(769)) == 5
    assert repack(packed=P(1032)) == 5
    assert repack(pbytes=1000) == 6
    assert repack() == 7


def test_missing_library_fails_loudly(monkeypatch):
    import w4a16_int4_weight_amd as mod
    monkeypatch.delenv("W4A16_LIBRARY", raising=False)
    monkeypatch.setattr(mod, "LIB_PATH", "/nonexistent/libw4a16.so")
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(ImportError):
        mod.w4a16_packed_bytes(512, 512, 128)
    with pytest.raises(ImportError):
        mod.lib
    # a library named through W4A16_LIBRARY that is missing is the same hard error
    monkeypatch.setattr(mod, "LIB_PATH", os.path.join(ROOT, "w4a16_int4_weight_amd", "libw4a16.so"))
    monkeypatch.setenv("W4A16_LIBRARY", "/nonexistent/libw4a16_other.so")
    with pytest.raises(ImportError):
        mod.w4a16_packed_bytes(512, 512, 128)


def test_build_module_and_binding_agree_on_library_path():
    import w4a16_int4_weight_amd as mod
    from w4a16_int4_weight_amd import build
    assert mod.LIB_PATH == build.LIB_PATH


def test_repack_gptq_validation_before_any_device_call(w):
    def repack(qw=P(256), qz=P(512), sc=P(768), dtype=1, K=512, N=512, G=128, packed=P(1024), pbytes=1 << 40):
        return w.lib.w4a16_repack_gptq(qw, qz, sc, dtype, K, N, G, packed, pbytes, None)
    assert repack(K=100) == 2
    assert repack(N=12) == 2
    assert repack(G=96) == 3
    assert repack(dtype=-1) == 4
    assert repack(qw=None) == 1
    assert repack(qz=None) == 1
    assert repack(sc=None) == 1
    assert repack(packed=None) == 1
    assert repack(qw=P(258)) == 5
    assert repack(sc=P(769)) == 5
    assert repack(packed=P(1032)) == 5
    assert repack(pbytes=1000) == 6
    assert repack() == 7


def test_embedding_validation_before_any_device_call(w):
    def emb(ids=P(256), T=4, packed=P(1024), pbytes=1 << 40, dtype=1, K=512, N=512, G=128, out=P(2048)):
        return w.lib.w4a16_embedding(ids, T, packed, pbytes, dtype, K, N, G, out, None)
    assert emb(K=100) == 2
    assert emb(N=12) == 2
    assert emb(G=96) == 3
    assert emb(dtype=2) == 4
    assert emb(T=-1) == 2
    assert emb(T=1 << 31) == 2
    assert emb(ids=None) == 1
    assert emb(packed=None) == 1
    assert emb(out=None) == 1
    assert emb(ids=P(258)) == 5
    assert emb(packed=P(1032)) == 5
    assert emb(out=P(2056)) == 5
    assert emb(pbytes=512 * 512 // 2) == 6
    # T = 0 is a valid no-op, even with NULL buffers
    assert emb(T=0, ids=None, packed=None, out=None) == 0
    # a fully valid call on this GPU-less host stops at the device check
    assert emb() == 7


def test_repack_columns_validation_before_any_device_call(w):
    for fn in (w.lib.w4a16_repack_columns, w.lib.w4a16_repack_gptq_columns):
        def rc(n0=0, nc=512, K=512, N=1024, G=128, qw=P(256), packed=P(1024), pbytes=1 << 40):
            return fn(qw, P(512), P(768), 1, K, N, G, n0, nc, packed, pbytes, None)
        assert rc(n0=8) == 2                    # not a whole block
        assert rc(nc=0) == 2
        assert rc(nc=12) == 2                   # not a multiple of 8
        assert rc(n0=512, nc=520) == 2          # past N
        assert rc(n0=0, nc=24) == 2             # half block not at the end
        assert rc(n0=-16) == 2
        assert rc(qw=None) == 1
        assert rc(pbytes=1000) == 6
        assert rc(n0=1000, nc=24, N=1024) == 2  # n0 not a whole block
        assert rc(n0=992, nc=24, N=1016) == 7   # last chunk ending in a half block: valid
        assert rc() == 7


def fnv1a64(data):
    h = 0xcbf29ce484222325
    for b in data:
        h = ((h ^ b) * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def test_packed_header_format(w):
    import struct
    import torch
    h = w.w4a16_packed_header(2048, 13288, 128, torch.bfloat16)
    assert len(h) == 64
    magic, version, dtype, K, N, G, nbytes, digest = struct.unpack("<8sIIqqqQQ", h[:56])
    assert magic == b"W4A16PK\0" and version == w.w4a16_layout_version() and dtype == 1
    assert (K, N, G) == (2048, 13288, 128) and nbytes == w.w4a16_packed_bytes(2048, 13288, 128)
    assert digest == fnv1a64(h[:48]) and h[56:] == bytes(8)
    assert w.w4a16_parse_packed_header(h) == (2048, 13288, 128, torch.bfloat16, nbytes)
    assert w.w4a16_parse_packed_header(w.w4a16_packed_header(512, 64, -1, torch.float16))[2:4] == (-1, torch.float16)


def test_packed_header_rejections(w):
    import struct
    import torch
    h = bytearray(w.w4a16_packed_header(1024, 272, 256, torch.bfloat16))
    for i in (0, 9, 20, 44, 50, 60):              # magic, version, K, size, hash, reserved
        bad = bytearray(h)
        bad[i] ^= 1
        with pytest.raises(w.W4A16Error) as e:
            w.w4a16_parse_packed_header(bad)
        assert e.value.status == "W4A16_ERR_LAYOUT"
    # another layout version with a consistent hash is still refused
    other = bytearray(h)
    struct.pack_into("<I", other, 8, w.w4a16_layout_version() + 1)
    struct.pack_into("<Q", other, 48, fnv1a64(bytes(other[:48])))
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_parse_packed_header(other)
    assert e.value.status == "W4A16_ERR_LAYOUT"
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_parse_packed_header(bytes(h[:40]))
    assert e.value.status == "W4A16_ERR_BUFFER_SIZE"
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_packed_header(1024, 270, 128, torch.bfloat16)
    assert e.value.status == "W4A16_ERR_SHAPE"


def test_save_and_load_packed_file_on_host(w, tmp_path):
    import torch
    K, N, G = 256, 40, 128
    nbytes = w.w4a16_packed_bytes(K, N, G)
    packed = torch.randint(0, 256, (nbytes,), dtype=torch.uint8)
    path = tmp_path / "layer.w4a16"
    w.save_packed(str(path), packed, K, N, G, torch.float16)
    raw = path.read_bytes()
    assert len(raw) == w.PAYLOAD_OFFSET + nbytes and raw[64:w.PAYLOAD_OFFSET] == bytes(w.PAYLOAD_OFFSET - 64)
    got, K2, N2, G2, dt = w.load_packed(str(path), device="cpu")
    assert (K2, N2, G2, dt) == (K, N, G, torch.float16) and torch.equal(got, packed)
    path.write_bytes(raw[:-1])                      # truncated payload
    with pytest.raises(w.W4A16Error):
        w.load_packed(str(path), device="cpu")


def test_w4a8_sizes(w):
    # codes, row scales and block sums, each from a 256-byte boundary
    for M, K in [(1, 2048), (512, 2048), (3, 384), (8, 6656)]:
        want = (M * K + 255) // 256 * 256 + (4 * M + 255) // 256 * 256 + 4 * M * (K // 128)
        assert w.w4a8_activation_bytes(M, K) == want
    for M, K in [(0, 2048), (-1, 2048), (4, 100), (4, 0)]:
        assert w.w4a8_activation_bytes(M, K) == 0
    # the same tiles and K split as the 16-bit MFMA GEMM; 32- and 64-row groups are not taken
    for M, K, N in [(16, 6656, 2048), (512, 2048, 131072), (1, 2048, 3072)]:
        assert w.w4a8_workspace_bytes(M, K, N, 128) == w.w4a16_workspace_bytes(M, K, N, 128)
    assert w.w4a8_workspace_bytes(16, 6656, 2048, 64) == 0


def test_w4a8_quantize_validation_before_any_device_call(w):
    def q(x=P(256), dtype=1, M=4, K=512, act=P(4096), abytes=1 << 30):
        return w.lib.w4a8_quantize(x, dtype, M, K, act, abytes, None)
    assert q(M=-1) == 2
    assert q(K=100) == 2
    assert q(K=(1 << 20) + 128) == 2
    assert q(dtype=2) == 4
    assert q(x=None) == 1
    assert q(act=None) == 1
    assert q(x=P(258)) == 5
    assert q(act=P(4100)) == 5
    assert q(abytes=4 * 512) == 6
    assert q(M=0, x=None, act=None) == 0
    assert q() == 7


def test_w4a8_gemm_validation_before_any_device_call(w):
    def g(act=P(256), abytes=1 << 30, packed=P(512), pbytes=1 << 40, dtype=1, y=P(1024), M=4, K=512, N=512,
          G=128, bias=None, ws=None, wsb=0):
        return w.lib.w4a8_gemm(act, abytes, packed, pbytes, dtype, y, M, K, N, G, bias, ws, wsb, None)
    assert g(M=-1) == 2
    assert g(K=500) == 2
    assert g(N=20) == 2
    assert g(G=96) == 3
    assert g(G=64) == 3
    assert g(G=32) == 3
    assert g(dtype=2) == 4
    assert g(act=None) == 1
    assert g(packed=None) == 1
    assert g(y=None) == 1
    assert g(act=P(264)) == 5
    assert g(bias=P(1025)) == 5
    assert g(abytes=512 * 4) == 6
    assert g(pbytes=512 * 512 // 2) == 6
    assert g(M=16, K=6656, N=2048) == 1                                 # K split: workspace needed
    assert g(M=16, K=6656, N=2048, ws=P(4096), wsb=64) == 6
    assert g(M=0, act=None, packed=None, y=None) == 0
    assert g(G=-1) == 7
    assert g() == 7
