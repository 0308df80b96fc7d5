"""MI355X (gfx950) hot path of a row-parallel block-scale fp8 linear layer.

Thin ctypes binding over ``libbsgemm.so`` (declared in ``include/bsgemm.h``):
the functions here only check and marshal torch tensors (device pointers,
sizes, the current HIP stream) and raise on a non-OK status.  Every step of
the path runs in the library's HIP kernels; there is no fallback.  If the
library has not been built, importing the functions raises immediately.

  bsgemm_fp8(A, a_scale, B, b_scale, C=None, bands=1, band_stride=0)
  band_reduce(parts, out=None)
  rowq_e4m3(x, q=None, scale=None)
  rowdq_e4m3(q, scale, y=None)
  blockq_e4m3(x, block_rows, q=None, scale=None)
  actq_e4m3(x, q=None, scale=None)
  bprepack_e4m3(B, Bp=None)
  bsgemm_fp8_pb(A, a_scale, Bp, b_scale, C=None, bands=1, band_stride=0)
  mxgemm_fp8(A, a_scale, B, b_scale, C=None, bands=1, band_stride=0)
  band_rowq_e4m3(parts, q=None, scale=None)
  mxq_e4m3(x, q=None, scale=None)

Tensors: e4m3 codes are uint8 (or torch.float8_e4m3fn, reinterpreted), bf16
values are torch.bfloat16 (or int16/uint16 bit patterns), scales float32.
All tensors must live on the current CUDA (HIP) device and be contiguous.
The C ABI receives raw pointers and cannot see sizes, so every wrapper checks
each operand's shape and each output's element count against the sizes the
call implies before it takes a pointer, and raises ValueError on a mismatch:
a wrong-shaped buffer never reaches a kernel.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbsgemm.so")

BS_OK, BS_ERR_INVALID, BS_ERR_UNSUPPORTED, BS_ERR_LAUNCH = 0, 1, 2, 3

# every extern "C" symbol of include/bsgemm.h
EXPORTS = ("bsgemm_fp8", "band_reduce", "rowq_e4m3", "rowdq_e4m3", "blockq_e4m3", "actq_e4m3",
           "mxgemm_fp8", "mxq_e4m3", "bprepack_e4m3", "bsgemm_fp8_pb", "band_rowq_e4m3",
           "bs_status_str")

_lib = None


class BSError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


def load():
    """Load libbsgemm.so (built in-tree by ``_build.py``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m block_scaled_fp8_bsgemm_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.bsgemm_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, vp]
    L.band_reduce.argtypes = [ctypes.POINTER(vp), i32, vp, i64, i64, vp]
    L.rowq_e4m3.argtypes = [vp, vp, vp, i64, i64, vp]
    L.rowdq_e4m3.argtypes = [vp, vp, vp, i64, i64, vp]
    L.blockq_e4m3.argtypes = [vp, vp, vp, i64, i64, i32, vp]
    L.actq_e4m3.argtypes = [vp, vp, vp, i64, i64, vp]
    L.mxgemm_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, vp]
    L.mxq_e4m3.argtypes = [vp, vp, vp, i64, i64, vp]
    L.bprepack_e4m3.argtypes = [vp, vp, i64, i64, vp]
    L.bsgemm_fp8_pb.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, vp]
    L.band_rowq_e4m3.argtypes = [ctypes.POINTER(vp), i32, vp, vp, i64, i64, vp]
    for f in ("bsgemm_fp8", "band_reduce", "rowq_e4m3", "rowdq_e4m3", "blockq_e4m3", "actq_e4m3",
              "mxgemm_fp8", "mxq_e4m3", "bprepack_e4m3", "bsgemm_fp8_pb", "band_rowq_e4m3"):
        getattr(L, f).restype = ctypes.c_int
    L.bs_status_str.argtypes = [ctypes.c_int]
    L.bs_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def status_str(status):
    return load().bs_status_str(int(status)).decode()


def _check(status, what):
    if status != BS_OK:
        raise BSError(status, what)


def _torch():
    import torch
    return torch


def _ptr(t, dtypes, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _shape(t, shape, name):
    _need(tuple(t.shape) == tuple(shape), f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _room(t, n, name):
    _need(t.numel() >= n, f"{name}: {t.numel()} elements, the call writes {n}")


def _dims2(t, name):
    _need(t.dim() == 2, f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape


def _band_elems(M, N, bands, band_stride):
    """elements of C the band epilogue writes (0 when the ABI will reject the
    band arguments anyway)"""
    if bands < 1 or M % bands or band_stride < 0:
        return 0
    band_rows = M // bands
    stride = band_stride if band_stride else band_rows * N
    return (bands - 1) * stride + band_rows * N


def _check_gemm_operands(A, a_scale, B, b_scale, kq, what):
    """A [M,K], B [N,K]; blockscale (kq = 128): a_scale [M,K/128], b_scale
    [N/128,K/128]; mxfp8 (kq = 32): a_scale [M,K/32], b_scale [N,K/32]."""
    M, K = _dims2(A, "A")
    N, K2 = _dims2(B, "B")
    _need(K2 == K, f"{what}: A is [M,{K}] but B is [N,{K2}]")
    _need(K % 128 == 0 and N % 128 == 0, f"{what}: K and N must be multiples of 128 (K={K}, N={N})")
    if kq == 128:
        _shape(a_scale, (M, K // 128), "a_scale")
        _shape(b_scale, (N // 128, K // 128), "b_scale")
    else:
        _shape(a_scale, (M, K // 32), "a_scale")
        _shape(b_scale, (N, K // 32), "b_scale")
    return M, N, K


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _u8():
    torch = _torch()
    return (torch.uint8, torch.int8, torch.float8_e4m3fn)


def _b16():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _f32():
    return (_torch().float32,)


def bsgemm_fp8(A, a_scale, B, b_scale, C=None, bands=1, band_stride=0, stream=None):
    """C (bf16) = blockscale(A [M,K] e4m3, a_scale [M,K/128]) x blockscale(B [N,K], b_scale [N/128,K/128])^T,
    written as `bands` destination-major row bands (band d at element d*band_stride)."""
    torch = _torch()
    M, N, K = _check_gemm_operands(A, a_scale, B, b_scale, 128, "bsgemm_fp8")
    need = _band_elems(M, N, bands, band_stride)
    if C is None:
        C = torch.empty(need, dtype=torch.bfloat16, device=A.device)
    _room(C, need, "C")
    st = load().bsgemm_fp8(_ptr(A, _u8(), "A"), _ptr(a_scale, _f32(), "a_scale"),
                           _ptr(B, _u8(), "B"), _ptr(b_scale, _f32(), "b_scale"),
                           _ptr(C, _b16(), "C"), M, N, K, bands, band_stride, _stream(stream))
    _check(st, "bsgemm_fp8")
    return C


def band_reduce(parts, out=None, stream=None):
    """out (bf16 [rows,N]) = bf16(sum_p fp32(parts[p])), parts summed in index order."""
    torch = _torch()
    parts = list(parts)
    _need(len(parts) >= 1, "band_reduce: no parts")
    rows, N = _dims2(parts[0], "parts[0]")
    for i, p in enumerate(parts):
        _shape(p, (rows, N), f"parts[{i}]")
    if out is None:
        out = torch.empty((rows, N), dtype=torch.bfloat16, device=parts[0].device)
    _room(out, rows * N, "out")
    ptrs = (ctypes.c_void_p * len(parts))(*[_ptr(p, _b16(), "part") for p in parts])
    st = load().band_reduce(ptrs, len(parts), _ptr(out, _b16(), "out"), rows, N, _stream(stream))
    _check(st, "band_reduce")
    return out


def rowq_e4m3(x, q=None, scale=None, stream=None):
    """(q uint8 [rows,N], scale fp32 [rows]) = per-row e4m3 quantization of bf16 x."""
    torch = _torch()
    rows, N = _dims2(x, "x")
    if q is None:
        q = torch.empty((rows, N), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _room(q, rows * N, "q")
    _room(scale, rows, "scale")
    st = load().rowq_e4m3(_ptr(x, _b16(), "x"), _ptr(q, _u8(), "q"), _ptr(scale, _f32(), "scale"),
                          rows, N, _stream(stream))
    _check(st, "rowq_e4m3")
    return q, scale


def rowdq_e4m3(q, scale, y=None, stream=None):
    """y (bf16 [rows,N]) = bf16(decode(q) * scale[row])."""
    torch = _torch()
    rows, N = _dims2(q, "q")
    _need(scale.numel() == rows, f"scale: {scale.numel()} elements for {rows} rows")
    if y is None:
        y = torch.empty((rows, N), dtype=torch.bfloat16, device=q.device)
    _room(y, rows * N, "y")
    st = load().rowdq_e4m3(_ptr(q, _u8(), "q"), _ptr(scale, _f32(), "scale"), _ptr(y, _b16(), "y"),
                           rows, N, _stream(stream))
    _check(st, "rowdq_e4m3")
    return y


def blockq_e4m3(x, block_rows, q=None, scale=None, stream=None):
    """(q uint8 [rows,cols], scale fp32 [ceil(rows/block_rows), cols/128]) for fp32 x."""
    torch = _torch()
    rows, cols = _dims2(x, "x")
    _need(block_rows in (1, 128), f"blockq_e4m3: block_rows must be 1 or 128, got {block_rows}")
    nscale = ((rows + block_rows - 1) // block_rows) * (cols // 128)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(((rows + block_rows - 1) // block_rows, cols // 128), dtype=torch.float32,
                            device=x.device)
    _room(q, rows * cols, "q")
    _room(scale, nscale, "scale")
    st = load().blockq_e4m3(_ptr(x, _f32(), "x"), _ptr(q, _u8(), "q"), _ptr(scale, _f32(), "scale"),
                            rows, cols, block_rows, _stream(stream))
    _check(st, "blockq_e4m3")
    return q, scale


def actq_e4m3(x, q=None, scale=None, stream=None):
    """(q uint8 [rows,cols], scale fp32 [rows, cols/128]) = 1x128 e4m3 quantization of bf16 x."""
    torch = _torch()
    rows, cols = _dims2(x, "x")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device)
    _room(q, rows * cols, "q")
    _room(scale, rows * (cols // 128), "scale")
    st = load().actq_e4m3(_ptr(x, _b16(), "x"), _ptr(q, _u8(), "q"), _ptr(scale, _f32(), "scale"),
                          rows, cols, _stream(stream))
    _check(st, "actq_e4m3")
    return q, scale


def mxgemm_fp8(A, a_scale, B, b_scale, C=None, bands=1, band_stride=0, stream=None):
    """C (bf16) = mx(A [M,K] e4m3, a_scale u8 [M,K/32]) x mx(B [N,K] e4m3, b_scale u8 [N,K/32])^T,
    E8M0 scales per 1x32 block, written as `bands` destination-major row bands."""
    torch = _torch()
    M, N, K = _check_gemm_operands(A, a_scale, B, b_scale, 32, "mxgemm_fp8")
    need = _band_elems(M, N, bands, band_stride)
    if C is None:
        C = torch.empty(need, dtype=torch.bfloat16, device=A.device)
    _room(C, need, "C")
    st = load().mxgemm_fp8(_ptr(A, _u8(), "A"), _ptr(a_scale, _u8(), "a_scale"),
                           _ptr(B, _u8(), "B"), _ptr(b_scale, _u8(), "b_scale"),
                           _ptr(C, _b16(), "C"), M, N, K, bands, band_stride, _stream(stream))
    _check(st, "mxgemm_fp8")
    return C


def mxq_e4m3(x, q=None, scale=None, stream=None):
    """(q uint8 [rows,cols], scale E8M0 uint8 [rows, cols/32]) = 1x32 mxfp8 quantization of bf16 x."""
    torch = _torch()
    rows, cols = _dims2(x, "x")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _room(q, rows * cols, "q")
    _room(scale, rows * (cols // 32), "scale")
    st = load().mxq_e4m3(_ptr(x, _b16(), "x"), _ptr(q, _u8(), "q"), _ptr(scale, _u8(), "scale"),
                         rows, cols, _stream(stream))
    _check(st, "mxq_e4m3")
    return q, scale


def bprepack_e4m3(B, Bp=None, stream=None):
    """Bp (uint8, N*K bytes) = the weight B [N,K] e4m3 in bsgemm_fp8_pb's operand order."""
    torch = _torch()
    N, K = _dims2(B, "B")
    if Bp is None:
        Bp = torch.empty(N * K, dtype=torch.uint8, device=B.device)
    _room(Bp, N * K, "Bp")
    st = load().bprepack_e4m3(_ptr(B, _u8(), "B"), _ptr(Bp, _u8(), "Bp"), N, K, _stream(stream))
    _check(st, "bprepack_e4m3")
    return Bp


def bsgemm_fp8_pb(A, a_scale, Bp, b_scale, C=None, bands=1, band_stride=0, stream=None):
    """bsgemm_fp8 with the weight prepacked by bprepack_e4m3 (Bp holds N*K bytes; N is
    taken from b_scale, [N/128, K/128])."""
    torch = _torch()
    M, K = _dims2(A, "A")
    _need(K % 128 == 0, f"bsgemm_fp8_pb: K must be a multiple of 128 (K={K})")
    _need(b_scale.dim() == 2 and b_scale.shape[1] == K // 128,
          f"b_scale: shape {tuple(b_scale.shape)}, expected [N/128, {K // 128}]")
    N = b_scale.shape[0] * 128
    _shape(a_scale, (M, K // 128), "a_scale")
    _need(Bp.numel() == N * K, f"Bp must hold N*K = {N * K} bytes, got {Bp.numel()}")
    need = _band_elems(M, N, bands, band_stride)
    if C is None:
        C = torch.empty(need, dtype=torch.bfloat16, device=A.device)
    _room(C, need, "C")
    st = load().bsgemm_fp8_pb(_ptr(A, _u8(), "A"), _ptr(a_scale, _f32(), "a_scale"),
                              _ptr(Bp, _u8(), "Bp"), _ptr(b_scale, _f32(), "b_scale"),
                              _ptr(C, _b16(), "C"), M, N, K, bands, band_stride, _stream(stream))
    _check(st, "bsgemm_fp8_pb")
    return C


def band_rowq_e4m3(parts, q=None, scale=None, stream=None):
    """(q uint8 [rows,N], scale fp32 [rows]) = rowq_e4m3(band_reduce(parts)) in one kernel."""
    torch = _torch()
    parts = list(parts)
    _need(len(parts) >= 1, "band_rowq_e4m3: no parts")
    rows, N = _dims2(parts[0], "parts[0]")
    for i, p in enumerate(parts):
        _shape(p, (rows, N), f"parts[{i}]")
    if q is None:
        q = torch.empty((rows, N), dtype=torch.uint8, device=parts[0].device)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=parts[0].device)
    _room(q, rows * N, "q")
    _room(scale, rows, "scale")
    ptrs = (ctypes.c_void_p * len(parts))(*[_ptr(p, _b16(), "part") for p in parts])
    st = load().band_rowq_e4m3(ptrs, len(parts), _ptr(q, _u8(), "q"), _ptr(scale, _f32(), "scale"),
                               rows, N, _stream(stream))
    _check(st, "band_rowq_e4m3")
    return q, scale
