"""Python binding of the MI355X W4A16 library (libw4a16.so): argument marshalling
only. Every step of the repack and the GEMM runs in the HIP kernels behind the C
ABI declared in include/w4a16.h; PyTorch provides device memory and streams.

Functions keep the C names:
  w4a16_layout_version()                         -> int
  w4a16_packed_bytes(K, N, group_size)           -> int (0 if unsupported)
  w4a16_workspace_bytes(M, K, N, group_size)     -> int
  w4a16_repack(qweight, qzeros, scales, group_size, packed=None, stream=None) -> packed uint8 tensor
  w4a16_repack_gptq(qweight, qzeros, scales, group_size, packed=None, stream=None) -> packed uint8 tensor
  w4a16_repack_columns / w4a16_repack_gptq_columns(qweight, qzeros, scales, N, n0, group_size, packed, stream)
      (one column chunk of the checkpoint into the whole weight's packed buffer)
  w4a16_packed_header(K, N, group_size, dtype) -> 64 bytes
  w4a16_parse_packed_header(header) -> (K, N, group_size, dtype, packed_bytes)
  w4a16_gemm(x, packed, N, group_size, bias=None, y=None, workspace=None, stream=None) -> y
      (workspace=None: a zero-filled per-device workspace is allocated on demand)
  w4a16_gemm_ex(..., path="auto"|"gemv"|"mfma", gemv_max_m=-1)            -> y
  w4a16_gemm_noalloc(x, packed, N, group_size, bias=None, y=None, stream=None) -> y
      (no workspace: the library's per-GPU scratch array; nothing is allocated when y is given)
  w4a16_embedding(ids, packed, K, N, group_size, dtype, out=None, stream=None) -> out [T, K]
  w4a16_status_str(code)                         -> str

Load-path helpers built on those calls (host-side data movement only):
  repack_from_host(qweight, qzeros, scales, group_size, fmt, chunk_columns, device)
      checkpoint tensors in host memory -> packed device buffer, one column chunk of
      the checkpoint on the device at a time
  save_packed(path, packed, K, N, group_size, dtype) / load_packed(path, device)
      a packed buffer on disk: the 64-byte header, zero padding to 64 KiB, the bytes

There is no fallback: if the library is missing, the first call (or access to
`lib`) raises ImportError; a call whose tensors are not on a gfx950 GPU returns the
library's error, raised here as W4A16Error.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a16.so")   # built by build.py

__all__ = [
    "W4A16Error", "lib", "w4a16_layout_version", "w4a16_packed_bytes", "w4a16_workspace_bytes",
    "w4a16_repack", "w4a16_repack_gptq", "w4a16_repack_columns", "w4a16_repack_gptq_columns",
    "w4a16_packed_header", "w4a16_parse_packed_header", "repack_from_host", "save_packed", "load_packed",
    "w4a16_gemm", "w4a16_gemm_ex", "w4a16_gemm_noalloc", "w4a16_embedding", "w4a16_status_str", "STATUS", "PATHS",
    "w4a16_stream_sink_bytes", "w4a16_stream_read", "w4a16_stream_copy", "w4a16_clock_stamp",
    "w4a16_wall_clock_hz",
]

STATUS = {
    0: "W4A16_OK", 1: "W4A16_ERR_NULL", 2: "W4A16_ERR_SHAPE", 3: "W4A16_ERR_GROUP",
    4: "W4A16_ERR_DTYPE", 5: "W4A16_ERR_ALIGN", 6: "W4A16_ERR_BUFFER_SIZE",
    7: "W4A16_ERR_DEVICE", 8: "W4A16_ERR_HIP", 9: "W4A16_ERR_PATH", 10: "W4A16_ERR_LAYOUT",
}
HEADER_BYTES = 64
PAYLOAD_OFFSET = 1 << 16       # packed bytes start 64 KiB into a saved file (page aligned)
DTYPES = {torch.float16: 0, torch.bfloat16: 1}
PATHS = {"auto": 0, "gemv": 1, "mfma": 2}


class W4A16Error(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        self.status = STATUS.get(code, str(code))
        super().__init__(f"{what}: {self.status} ({w4a16_status_str(code)})")


_lib = None


def _load():
    """Loads libw4a16.so on first use. There is no fallback: a missing library is an
    error the caller sees, never a silent switch to another implementation."""
    global _lib
    if _lib is not None:
        return _lib
    # W4A16_LIBRARY names another build of the same library (the host-sanitized one the
    # CPU tests load); a missing file is the same hard error
    path = os.environ.get("W4A16_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m w4a16_int4_weight_amd.build` "
                          "(the W4A16 path has no fallback)")
    h = ctypes.CDLL(path)
    _vp, _i64, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    h.w4a16_layout_version.argtypes = []
    h.w4a16_layout_version.restype = _int
    h.w4a16_packed_bytes.argtypes = [_i64, _i64, _i64]
    h.w4a16_packed_bytes.restype = _sz
    h.w4a16_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
    h.w4a16_workspace_bytes.restype = _sz
    h.w4a16_repack.argtypes = [_vp, _vp, _vp, _int, _i64, _i64, _i64, _vp, _sz, _vp]
    h.w4a16_repack.restype = _int
    h.w4a16_repack_gptq.argtypes = h.w4a16_repack.argtypes
    h.w4a16_repack_gptq.restype = _int
    h.w4a16_repack_columns.argtypes = [_vp, _vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _vp, _sz, _vp]
    h.w4a16_repack_columns.restype = _int
    h.w4a16_repack_gptq_columns.argtypes = h.w4a16_repack_columns.argtypes
    h.w4a16_repack_gptq_columns.restype = _int
    h.w4a16_packed_header.argtypes = [_i64, _i64, _i64, _int, _vp, _sz]
    h.w4a16_packed_header.restype = _int
    _p64 = ctypes.POINTER(ctypes.c_int64)
    h.w4a16_parse_packed_header.argtypes = [_vp, _sz, _p64, _p64, _p64, ctypes.POINTER(ctypes.c_int),
                                            ctypes.POINTER(ctypes.c_size_t)]
    h.w4a16_parse_packed_header.restype = _int
    h.w4a16_gemm.argtypes = [_vp, _vp, _sz, _int, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _sz, _vp]
    h.w4a16_gemm.restype = _int
    h.w4a16_gemm_ex.argtypes = h.w4a16_gemm.argtypes + [_int, _i64]
    h.w4a16_gemm_ex.restype = _int
    h.w4a16_gemm_noalloc.argtypes = [_vp, _vp, _sz, _int, _vp, _i64, _i64, _i64, _i64, _vp, _vp]
    h.w4a16_gemm_noalloc.restype = _int
    h.w4a16_embedding.argtypes = [_vp, _i64, _vp, _sz, _int, _i64, _i64, _i64, _vp, _vp]
    h.w4a16_embedding.restype = _int
    h.w4a8_activation_bytes.argtypes = [_i64, _i64]
    h.w4a8_activation_bytes.restype = _sz
    h.w4a8_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
    h.w4a8_workspace_bytes.restype = _sz
    h.w4a8_quantize.argtypes = [_vp, _int, _i64, _i64, _vp, _sz, _vp]
    h.w4a8_quantize.restype = _int
    h.w4a8_gemm.argtypes = [_vp, _sz, _vp, _sz, _int, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _sz, _vp]
    h.w4a8_gemm.restype = _int
    h.w4a16_stream_sink_bytes.argtypes = [_sz]
    h.w4a16_stream_sink_bytes.restype = _sz
    h.w4a16_stream_read.argtypes = [_vp, _sz, _vp, _sz, _vp]
    h.w4a16_stream_read.restype = _int
    h.w4a16_stream_copy.argtypes = [_vp, _vp, _sz, _vp]
    h.w4a16_stream_copy.restype = _int
    h.w4a16_clock_stamp.argtypes = [_vp, _vp]
    h.w4a16_clock_stamp.restype = _int
    h.w4a16_wall_clock_hz.argtypes = [ctypes.POINTER(_i64)]
    h.w4a16_wall_clock_hz.restype = _int
    h.w4a16_status_str.argtypes = [_int]
    h.w4a16_status_str.restype = ctypes.c_char_p
    _lib = h
    return h


def __getattr__(name):
    # `lib` is the loaded library handle, loaded on first access
    if name == "lib":
        return _load()
    raise AttributeError(name)


def w4a16_status_str(code):
    return _load().w4a16_status_str(int(code)).decode()


def w4a16_layout_version():
    return _load().w4a16_layout_version()


def w4a16_packed_bytes(K, N, group_size):
    return _load().w4a16_packed_bytes(K, N, group_size)


def w4a16_workspace_bytes(M, K, N, group_size):
    return _load().w4a16_workspace_bytes(M, K, N, group_size)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(code, what):
    if code != 0:
        raise W4A16Error(code, what)


def _dtype_code(dtype):
    if dtype not in DTYPES:
        raise W4A16Error(4, f"dtype {dtype}")
    return DTYPES[dtype]


def w4a16_repack(qweight, qzeros, scales, group_size=128, packed=None, stream=None):
    """AWQ qweight int32 [K, N/8], qzeros int32 [K/G, N/8], scales [K/G, N] (fp16/bf16),
    all on one GPU -> packed uint8 tensor of w4a16_packed_bytes(K, N, group_size) bytes."""
    K, N = qweight.shape[0], qweight.shape[1] * 8
    nbytes = w4a16_packed_bytes(K, N, group_size)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qweight.device)
    for t, name in ((qweight, "qweight"), (qzeros, "qzeros"), (scales, "scales")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise ValueError("qweight and qzeros must be int32")
    G = K if group_size == -1 else group_size
    if G > 0 and K % G == 0 and (tuple(qzeros.shape) != (K // G, N // 8) or tuple(scales.shape) != (K // G, N)):
        raise ValueError("qzeros must be [K/G, N/8] and scales [K/G, N]")
    code = _load().w4a16_repack(_ptr(qweight), _ptr(qzeros), _ptr(scales), _dtype_code(scales.dtype),
                            K, N, group_size, _ptr(packed), packed.numel() * packed.element_size(),
                            _stream(stream, qweight.device))
    _check(code, "w4a16_repack")
    return packed


def w4a16_repack_gptq(qweight, qzeros, scales, group_size=128, packed=None, stream=None):
    """GPTQ-standard qweight int32 [K/8, N] (codes along K), qzeros int32 [K/G, N/8]
    (standard order along N), scales [K/G, N] -> the same packed buffer as w4a16_repack."""
    K, N = qweight.shape[0] * 8, qweight.shape[1]
    nbytes = w4a16_packed_bytes(K, N, group_size)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qweight.device)
    for t, name in ((qweight, "qweight"), (qzeros, "qzeros"), (scales, "scales")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise ValueError("qweight and qzeros must be int32")
    G = K if group_size == -1 else group_size
    if G > 0 and K % G == 0 and (tuple(qzeros.shape) != (K // G, N // 8) or tuple(scales.shape) != (K // G, N)):
        raise ValueError("qzeros must be [K/G, N/8] and scales [K/G, N]")
    code = _load().w4a16_repack_gptq(_ptr(qweight), _ptr(qzeros), _ptr(scales), _dtype_code(scales.dtype),
                                     K, N, group_size, _ptr(packed), packed.numel() * packed.element_size(),
                                     _stream(stream, qweight.device))
    _check(code, "w4a16_repack_gptq")
    return packed


def _repack_columns(fn, name, qweight, qzeros, scales, K, N, n0, nc, group_size, packed, stream):
    for t, tname in ((qweight, "qweight"), (qzeros, "qzeros"), (scales, "scales")):
        if not t.is_contiguous():
            raise ValueError(f"{tname} must be contiguous")
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise ValueError("qweight and qzeros must be int32")
    code = fn(_ptr(qweight), _ptr(qzeros), _ptr(scales), _dtype_code(scales.dtype), K, N, group_size, n0, nc,
              _ptr(packed), packed.numel() * packed.element_size(), _stream(stream, qweight.device))
    _check(code, name)
    return packed


def w4a16_repack_columns(qweight, qzeros, scales, N, n0, group_size=128, packed=None, stream=None):
    """AWQ tensors of columns [n0, n0 + nc) (qweight int32 [K, nc/8], qzeros [K/G, nc/8],
    scales [K/G, nc]) -> those columns of the K x N weight's packed buffer."""
    K, nc = qweight.shape[0], qweight.shape[1] * 8
    if packed is None:
        packed = torch.empty(max(w4a16_packed_bytes(K, N, group_size), 1), dtype=torch.uint8, device=qweight.device)
    return _repack_columns(_load().w4a16_repack_columns, "w4a16_repack_columns", qweight, qzeros, scales, K, N,
                           n0, nc, group_size, packed, stream)


def w4a16_repack_gptq_columns(qweight, qzeros, scales, N, n0, group_size=128, packed=None, stream=None):
    """GPTQ-standard tensors of columns [n0, n0 + nc) (qweight int32 [K/8, nc], qzeros
    [K/G, nc/8], scales [K/G, nc]) -> those columns of the K x N weight's packed buffer."""
    K, nc = qweight.shape[0] * 8, qweight.shape[1]
    if packed is None:
        packed = torch.empty(max(w4a16_packed_bytes(K, N, group_size), 1), dtype=torch.uint8, device=qweight.device)
    return _repack_columns(_load().w4a16_repack_gptq_columns, "w4a16_repack_gptq_columns", qweight, qzeros, scales,
                           K, N, n0, nc, group_size, packed, stream)


def repack_from_host(qweight, qzeros, scales, group_size=128, fmt="awq", chunk_columns=4096, device="cuda:0",
                     stream=None):
    """Checkpoint tensors in host memory -> packed device buffer. Column chunks of
    `chunk_columns` (a multiple of 16) are copied to the device and repacked one at a
    time, so the device holds one chunk of the checkpoint tensors besides the packed
    buffer. fmt "awq": qweight [K, N/8]; "gptq": qweight [K/8, N] (codes along K)."""
    if fmt not in ("awq", "gptq"):
        raise ValueError(f"fmt {fmt!r}")
    if chunk_columns <= 0 or chunk_columns % 16 != 0:
        raise ValueError("chunk_columns must be a positive multiple of 16")
    K, N = (qweight.shape[0], qweight.shape[1] * 8) if fmt == "awq" else (qweight.shape[0] * 8, qweight.shape[1])
    nbytes = w4a16_packed_bytes(K, N, group_size)
    if nbytes == 0:
        raise W4A16Error(2, "repack_from_host")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
    for n0 in range(0, N, chunk_columns):
        nc = min(chunk_columns, N - n0)
        w0, w1 = n0 // 8, (n0 + nc) // 8
        qw = qweight[:, w0:w1] if fmt == "awq" else qweight[:, n0:n0 + nc]
        qw = qw.contiguous().to(device)
        qz = qzeros[:, w0:w1].contiguous().to(device)
        sc = scales[:, n0:n0 + nc].contiguous().to(device)
        if fmt == "awq":
            w4a16_repack_columns(qw, qz, sc, N, n0, group_size, packed, stream)
        else:
            w4a16_repack_gptq_columns(qw, qz, sc, N, n0, group_size, packed, stream)
        del qw, qz, sc
    return packed


def w4a16_packed_header(K, N, group_size, dtype):
    """The 64-byte header of a stored packed buffer (bytes)."""
    buf = ctypes.create_string_buffer(HEADER_BYTES)
    _check(_load().w4a16_packed_header(K, N, group_size, _dtype_code(dtype), buf, HEADER_BYTES),
           "w4a16_packed_header")
    return buf.raw


def w4a16_parse_packed_header(header):
    """bytes -> (K, N, group_size, torch dtype, packed_bytes); W4A16Error if invalid."""
    header = bytes(header)
    K, N, G = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    dt, nbytes = ctypes.c_int(), ctypes.c_size_t()
    _check(_load().w4a16_parse_packed_header(header, len(header), ctypes.byref(K), ctypes.byref(N),
                                             ctypes.byref(G), ctypes.byref(dt), ctypes.byref(nbytes)),
           "w4a16_parse_packed_header")
    dtype = {v: k for k, v in DTYPES.items()}[dt.value]
    return K.value, N.value, G.value, dtype, nbytes.value


def save_packed(path, packed, K, N, group_size, dtype):
    """Writes the header, zero padding to 64 KiB and the packed bytes."""
    header = w4a16_packed_header(K, N, group_size, dtype)
    nbytes = w4a16_packed_bytes(K, N, group_size)
    if packed.numel() * packed.element_size() < nbytes:
        raise W4A16Error(6, "save_packed")
    data = packed.reshape(-1).view(torch.uint8)[:nbytes].cpu().numpy().tobytes()
    with open(path, "wb") as f:
        f.write(header + bytes(PAYLOAD_OFFSET - HEADER_BYTES))
        f.write(data)


def load_packed(path, device="cuda:0"):
    """-> (packed device tensor, K, N, group_size, dtype). W4A16Error (W4A16_ERR_LAYOUT)
    if the file was written for another layout version or is damaged: repack from the
    checkpoint instead."""
    with open(path, "rb") as f:
        head = f.read(PAYLOAD_OFFSET)
        K, N, G, dtype, nbytes = w4a16_parse_packed_header(head[:HEADER_BYTES])
        if len(head) != PAYLOAD_OFFSET or any(head[HEADER_BYTES:]):
            raise W4A16Error(10, "load_packed")
        data = f.read(nbytes)
        if len(data) != nbytes or f.read(1):
            raise W4A16Error(10, "load_packed")
    packed = torch.frombuffer(bytearray(data), dtype=torch.uint8).to(device)
    return packed, K, N, G, dtype


_workspaces = {}


def _default_workspace(device, nbytes, stream=None):
    """A zero-filled workspace per (device, stream), grown on demand. The kernels leave
    its counters at zero, so consecutive calls on one stream reuse it; calls on other
    streams get their own. It is allocated and zeroed on that stream, so the memory of
    a buffer replaced by a larger one is only handed out again behind the calls already
    queued there."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    key = (torch.device(device).index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _gemm_args(x, packed, N, group_size, bias, y, workspace, stream):
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    M, K = x.shape
    if workspace is None and M > 0:
        need = w4a16_workspace_bytes(M, K, N, group_size)
        if need > 0:
            workspace = _default_workspace(x.device, need, stream)
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if tuple(y.shape) != (M, N) or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("y must be a contiguous [M, N] tensor of x's dtype")
    if bias is not None and (bias.dtype != x.dtype or tuple(bias.shape) != (N,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [N] tensor of x's dtype")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _ptr(packed), packed.numel() * packed.element_size(), _dtype_code(x.dtype),
            _ptr(y), M, K, N, group_size, _ptr(bias), _ptr(workspace), ws_bytes, _stream(stream, x.device))
    return args, y


def w4a16_gemm(x, packed, N, group_size=128, bias=None, y=None, workspace=None, stream=None):
    """x [M, K] (fp16/bf16) times the packed weight (+ bias) -> y [M, N] of x's dtype."""
    args, y = _gemm_args(x, packed, N, group_size, bias, y, workspace, stream)
    _check(_load().w4a16_gemm(*args), "w4a16_gemm")
    return y


def w4a16_gemm_ex(x, packed, N, group_size=128, bias=None, y=None, workspace=None, stream=None,
                  path="auto", gemv_max_m=-1):
    """w4a16_gemm with the kernel path forced ("auto", "gemv" or "mfma")."""
    if path not in PATHS:
        raise W4A16Error(9, f"path {path!r}")
    args, y = _gemm_args(x, packed, N, group_size, bias, y, workspace, stream)
    _check(_load().w4a16_gemm_ex(*args, PATHS[path], gemv_max_m), "w4a16_gemm_ex")
    return y


def w4a16_gemm_noalloc(x, packed, N, group_size=128, bias=None, y=None, stream=None):
    """w4a16_gemm without a workspace: the library's own per-GPU scratch array holds
    the K-split partials (calls that may overlap in time on one GPU must not be made).
    y must be given by a caller that cannot allocate."""
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if tuple(y.shape) != (M, N) or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("y must be a contiguous [M, N] tensor of x's dtype")
    if bias is not None and (bias.dtype != x.dtype or tuple(bias.shape) != (N,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [N] tensor of x's dtype")
    code = _load().w4a16_gemm_noalloc(_ptr(x), _ptr(packed), packed.numel() * packed.element_size(),
                                      _dtype_code(x.dtype), _ptr(y), M, K, N, group_size, _ptr(bias),
                                      _stream(stream, x.device))
    _check(code, "w4a16_gemm_noalloc")
    return y


NOALLOC_SCRATCH_BYTES = 4 << 20      # W4A16_NOALLOC_SCRATCH_BYTES


def w4a16_embedding(ids, packed, K, N, group_size=128, dtype=torch.bfloat16, out=None, stream=None):
    """Token ids int32 [T] -> out [T, K] of `dtype`: row i is column ids[i] of the
    dequantised head weight the packed buffer holds (zeros for ids outside [0, N))."""
    if ids.dim() != 1 or ids.dtype != torch.int32 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 [T] tensor")
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, K), dtype=dtype, device=ids.device)
    if tuple(out.shape) != (T, K) or out.dtype != dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, K] tensor of `dtype`")
    code = _load().w4a16_embedding(_ptr(ids), T, _ptr(packed), packed.numel() * packed.element_size(),
                                   _dtype_code(dtype), K, N, group_size, _ptr(out), _stream(stream, ids.device))
    _check(code, "w4a16_embedding")
    return out


# ---------------------------------------------------------------- W4A8

def w4a8_activation_bytes(M, K):
    return int(_load().w4a8_activation_bytes(M, K))


def w4a8_workspace_bytes(M, K, N, group_size):
    return int(_load().w4a8_workspace_bytes(M, K, N, group_size))


def w4a8_act_parts(act, M, K):
    """Views of a W4A8 activation buffer: (codes uint8 [M, K] in operand order,
    row scales float32 [M], block sums float32 [M, K / 128])."""
    off_s = (M * K + 255) // 256 * 256
    off_b = off_s + (M * 4 + 255) // 256 * 256
    codes = act[:M * K].view(M, K)
    scale = act[off_s:off_s + 4 * M].view(torch.float32)
    sums = act[off_b:off_b + 4 * M * (K // 128)].view(torch.float32).view(M, K // 128)
    return codes, scale, sums


def w4a8_quantize(x, act=None, stream=None):
    """x [M, K] (fp16/bf16) -> W4A8 activation buffer (uint8 tensor of
    w4a8_activation_bytes(M, K) bytes; see w4a8_act_parts for its parts)."""
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    M, K = x.shape
    need = w4a8_activation_bytes(M, K) if M > 0 else 0
    if act is None:
        act = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    code = _load().w4a8_quantize(_ptr(x), _dtype_code(x.dtype), M, K, _ptr(act), act.numel() * act.element_size(),
                                 _stream(stream, x.device))
    _check(code, "w4a8_quantize")
    return act


def w4a8_gemm(act, packed, M, K, N, group_size=128, dtype=torch.bfloat16, bias=None, y=None, workspace=None,
              stream=None):
    """W4A8 activation buffer (from w4a8_quantize) times the packed weight (+ bias)
    -> y [M, N] of `dtype` (the dtype of the weight's scales)."""
    if workspace is None and M > 0:
        need = w4a8_workspace_bytes(M, K, N, group_size)
        if need > 0:
            workspace = _default_workspace(act.device, need, stream)
    if y is None:
        y = torch.empty((M, N), dtype=dtype, device=act.device)
    if tuple(y.shape) != (M, N) or y.dtype != dtype or not y.is_contiguous():
        raise ValueError("y must be a contiguous [M, N] tensor of `dtype`")
    if bias is not None and (bias.dtype != dtype or tuple(bias.shape) != (N,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [N] tensor of `dtype`")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = _load().w4a8_gemm(_ptr(act), act.numel() * act.element_size(), _ptr(packed),
                             packed.numel() * packed.element_size(), _dtype_code(dtype), _ptr(y), M, K, N, group_size,
                             _ptr(bias), _ptr(workspace), ws_bytes, _stream(stream, act.device))
    _check(code, "w4a8_gemm")
    return y


def w4a8_linear(x, packed, N, group_size=128, bias=None, y=None, act=None, workspace=None, stream=None):
    """x [M, K] (fp16/bf16): quantise to fp8 per row, then the W4A8 product -> y [M, N]."""
    M, K = x.shape
    act = w4a8_quantize(x, act=act, stream=stream)
    return w4a8_gemm(act, packed, M, K, N, group_size, x.dtype, bias, y, workspace, stream)


# ---------------------------------------------------------------- streaming references
# (include/w4a16_measure.h: the achievable-bandwidth floor beside the HBM-bound rows)

def w4a16_stream_sink_bytes(nbytes):
    return int(_load().w4a16_stream_sink_bytes(nbytes))


def w4a16_stream_read(src, nbytes=None, sink=None, stream=None):
    """Reads the first `nbytes` bytes of the device tensor `src` once; returns the sink
    (uint8, 16 bytes per workgroup: each workgroup's XOR of what it read)."""
    total = src.numel() * src.element_size()
    nbytes = total if nbytes is None else nbytes
    if nbytes > total:
        raise ValueError("nbytes exceeds the tensor")
    need = w4a16_stream_sink_bytes(nbytes) if nbytes else 0
    if sink is None:
        sink = torch.empty(max(need, 16), dtype=torch.uint8, device=src.device)
    _check(_load().w4a16_stream_read(_ptr(src), nbytes, _ptr(sink), sink.numel() * sink.element_size(),
                                     _stream(stream, src.device)), "w4a16_stream_read")
    return sink


def w4a16_clock_stamp(dst, index=0, stream=None):
    """Stores the GPU's wall clock, when the launch runs, into dst[index] (dst: an int64
    device tensor); capturable in a HIP graph. Ticks per second: w4a16_wall_clock_hz()."""
    if dst.dtype != torch.int64 or not 0 <= index < dst.numel() or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous int64 tensor holding `index`")
    _check(_load().w4a16_clock_stamp(ctypes.c_void_p(dst.data_ptr() + 8 * index), _stream(stream, dst.device)),
           "w4a16_clock_stamp")


def w4a16_wall_clock_hz():
    hz = ctypes.c_int64(0)
    _check(_load().w4a16_wall_clock_hz(ctypes.byref(hz)), "w4a16_wall_clock_hz")
    return int(hz.value)


def w4a16_stream_copy(src, dst, nbytes=None, stream=None):
    """Copies the first `nbytes` bytes of `src` into `dst` (device tensors)."""
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    if nbytes > src.numel() * src.element_size() or nbytes > dst.numel() * dst.element_size():
        raise ValueError("nbytes exceeds a tensor")
    _check(_load().w4a16_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream, src.device)),
           "w4a16_stream_copy")
    return dst
