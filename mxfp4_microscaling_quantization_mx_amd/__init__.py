"""MI355X-native MXFP4 (OCP MX v1.0) quantizer and block-scaled GEMMs.

A thin ctypes binding over ``libmxfp4.so`` (declared in ``include/mx.h``).
PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  The binding only allocates
output tensors and marshals pointers, shapes and strides.  If the library is
missing, every call raises: there is no fallback path.

    q = quantize(x, axis="last", block="1d", rounding="rne", rht_mask=None)
    y = dequantize(q, torch.float32)
    qt = transpose(q2d)                                 # exact, 2-D blocks only
    c = gemm(qa, qb, torch.bfloat16)                    # C = A * B^T
    c = grouped_gemm(qa, offsets, qb_stacked, torch.bfloat16)
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxfp4.so")

MX_OK, MX_ERR_INVALID_ARG, MX_ERR_UNSUPPORTED, MX_ERR_HIP = 0, 1, 2, 3
MX_DT_F32, MX_DT_BF16 = 0, 1
_AXIS = {"last": 0, "dim0": 1}
_BLOCK = {"1d": 0, "2d": 1}
_ROUND = {"rne": 0, "sr": 1, "sr8": 2}
_SCALE = {"floor": 0, "round_up": 1, "prescale_3_4": 2}
# MX element types: name -> (mx_elem, bits per element)
_ELEM = {"e2m1": (0, 4), "e4m3": (1, 8), "e5m2": (2, 8), "e2m3": (3, 6), "e3m2": (4, 6)}
_DTYPE = {torch.float32: MX_DT_F32, torch.bfloat16: MX_DT_BF16}

EXPORTED = ("mx_quantize", "mx_quantize_gather", "mx_quantize_scatter", "mx_dequantize", "mx_transpose", "mx_gemm",
            "mx_gemm_quantize", "mx_gemm_workspace_size", "mx_gemm_noalloc", "mx_gemm_fused_quant_a", "mx_grouped_gemm",
            "mx_grouped_gemm_quantize", "mx_clip_count",
            "mx_last_error", "mx_version")


class MxTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("K", ctypes.c_int64),
                ("ld_codes", ctypes.c_int64), ("ld_scales", ctypes.c_int64),
                ("block", ctypes.c_int32), ("elem", ctypes.c_int32)]


class QuantCfgC(ctypes.Structure):
    _fields_ = [("axis", ctypes.c_int32), ("block", ctypes.c_int32),
                ("rounding", ctypes.c_int32), ("use_rht", ctypes.c_int32),
                ("rht_sign_mask", ctypes.c_uint32), ("scale_mode", ctypes.c_uint32),
                ("philox_seed", ctypes.c_uint64), ("philox_offset", ctypes.c_uint64)]


class MXError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libmxfp4 status {status}: {msg}")
        self.status = status


_lib = None


def load_library(path=LIB_PATH):
    """Load libmxfp4.so and declare its signatures (no GPU is touched)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m mxfp4_microscaling_quantization_mx_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    PT = ctypes.POINTER(MxTensorC)
    lib.mx_quantize.argtypes = [P, I32, I64, I64, I64, ctypes.POINTER(QuantCfgC), PT, P]
    lib.mx_quantize_gather.argtypes = [P, I32, I64, I64, I64, P, I64, ctypes.POINTER(QuantCfgC), PT, P]
    lib.mx_quantize_scatter.argtypes = [P, I32, I64, I64, I64, P, I32, ctypes.POINTER(QuantCfgC), PT, P]
    lib.mx_dequantize.argtypes = [PT, I32, U32, P, I32, I64, P]
    lib.mx_transpose.argtypes = [PT, PT, P]
    lib.mx_gemm.argtypes = [PT, PT, P, I32, I64, P, ctypes.c_size_t, P]
    lib.mx_gemm_quantize.argtypes = [PT, PT, I32, PT, P]
    lib.mx_gemm_noalloc.argtypes = [PT, PT, P, I32, I64, P]
    lib.mx_gemm_fused_quant_a.argtypes = [P, I32, I64, I64, I64, ctypes.POINTER(QuantCfgC), PT, P, I32, I64, P]
    lib.mx_gemm_workspace_size.argtypes = [I64, I64, I64]
    lib.mx_gemm_workspace_size.restype = ctypes.c_size_t
    lib.mx_grouped_gemm.argtypes = [PT, P, I32, PT, I64, I64, P, I32, I64, P]
    lib.mx_grouped_gemm_quantize.argtypes = [PT, P, I32, PT, I64, I64, I32, PT, P]
    lib.mx_clip_count.argtypes = [P, I32, I64, I64, I64, ctypes.POINTER(QuantCfgC), I32, P, P]
    for f in ("mx_quantize", "mx_quantize_gather", "mx_quantize_scatter", "mx_dequantize", "mx_transpose", "mx_gemm",
              "mx_gemm_quantize", "mx_gemm_noalloc", "mx_gemm_fused_quant_a", "mx_grouped_gemm",
              "mx_grouped_gemm_quantize"):
        getattr(lib, f).restype = ctypes.c_int
    lib.mx_last_error.restype = ctypes.c_char_p
    lib.mx_last_error.argtypes = []
    lib.mx_version.restype = ctypes.c_char_p
    lib.mx_version.argtypes = []
    _lib = lib
    return lib


def _check(status):
    if status != MX_OK:
        raise MXError(status, _lib.mx_last_error().decode())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


@dataclass
class MXTensor:
    """K-major MX operand: codes uint8 [rows, K*bits/8] (MXFP4: K/2), scales
    uint8 [rows, K/32] (1-D) or [rows/32, K/32] (2-D).  Row strides are taken
    from the tensors.  elem: "e2m1" (MXFP4), "e4m3"/"e5m2" (MXFP8) or
    "e2m3"/"e3m2" (MXFP6)."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    K: int
    block: str = "1d"
    elem: str = "e2m1"

    def c_struct(self):
        return MxTensorC(self.codes.data_ptr(), self.scales.data_ptr(), self.rows, self.K,
                         self.codes.stride(0) if self.codes.dim() == 2 else self.K * _ELEM[self.elem][1] // 8,
                         self.scales.stride(0) if self.scales.dim() == 2 else self.K // 32,
                         _BLOCK[self.block], _ELEM[self.elem][0])


def empty_mx(rows, K, block="1d", device="cuda", experts=None, elem="e2m1"):
    """Allocate an uninitialised MX operand (codes + scales) on `device`.

    Code rows are padded to a multiple of 128 bytes and scale rows to a
    multiple of 16 bytes (the row strides are carried in the tensors), so the
    GEMMs' row segments start on cache-line boundaries and their scale fetches
    are aligned.  With `experts=E` the tensors get a leading expert dimension
    (the stacked weights of grouped_gemm); expert e is `expert(q, e)`."""
    srows = rows // 32 if block == "2d" else rows
    lead = () if experts is None else (experts,)
    cb = K * _ELEM[elem][1] // 8
    ldc = (cb + 127) // 128 * 128
    codes = torch.empty(lead + (rows, ldc), dtype=torch.uint8, device=device)[..., :cb]
    ld = (K // 32 + 15) // 16 * 16
    scales = torch.empty(lead + (srows, ld), dtype=torch.uint8, device=device)[..., :K // 32]
    return MXTensor(codes, scales, rows, K, block, elem)


def expert(q, e):
    """View of expert e of a stacked operand from empty_mx(..., experts=E)."""
    return MXTensor(q.codes[e], q.scales[e], q.rows, q.K, q.block, q.elem)


def quantize(x, axis="last", block="1d", rounding="rne", rht_mask=None, seed=0, offset=0,
             out=None, scale_mode="floor", elem="e2m1"):
    """Quantize a 2-D bf16/fp32 CUDA tensor to MXFP4 (or, with elem, MXFP8 /
    MXFP6; see mx_quantize in include/mx.h).

    axis="dim0" blocks along dim 0 and returns the quantized transpose.
    scale_mode: "floor" (the reference rule), "round_up" or "prescale_3_4".
    With `out` given, its element type is the one produced."""
    lib = load_library()
    if x.dim() != 2 or x.dtype not in _DTYPE or not x.is_cuda:
        raise ValueError("quantize expects a 2-D bf16/float32 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("quantize expects a row-major tensor (stride(1) == 1)")
    R, C = x.shape
    rows, K = (C, R) if axis == "dim0" else (R, C)
    if out is None:
        out = empty_mx(rows, K, block, x.device, elem=elem)
    cfg = QuantCfgC(_AXIS[axis], _BLOCK[block], _ROUND[rounding], int(rht_mask is not None),
                    (rht_mask or 0) & 0xFFFFFFFF, _SCALE[scale_mode], seed & (2**64 - 1),
                    offset & (2**64 - 1))
    ot = out.c_struct()
    _check(lib.mx_quantize(_ptr(x), _DTYPE[x.dtype], R, C, x.stride(0), ctypes.byref(cfg),
                           ctypes.byref(ot), _stream(x)))
    return out


def clip_count(x, axis="last", block="1d", rht_mask=None, scale_mode="floor", elem="e2m1", out=None):
    """Clipping statistic of quantizing x with these settings: the number of
    elements that saturate at the element type's largest normal (see
    mx_clip_count in include/mx.h).  Returns a one-element int64 CUDA tensor;
    with `out` given (one int64 element), the count is added to it."""
    lib = load_library()
    if x.dim() != 2 or x.dtype not in _DTYPE or not x.is_cuda:
        raise ValueError("clip_count expects a 2-D bf16/float32 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("clip_count expects a row-major tensor (stride(1) == 1)")
    if out is None:
        out = torch.zeros(1, dtype=torch.int64, device=x.device)
    elif out.dtype != torch.int64 or out.numel() != 1 or not out.is_cuda:
        raise ValueError("clip_count: out must be a one-element int64 CUDA tensor")
    R, C = x.shape
    cfg = QuantCfgC(_AXIS[axis], _BLOCK[block], _ROUND["rne"], int(rht_mask is not None),
                    (rht_mask or 0) & 0xFFFFFFFF, _SCALE[scale_mode], 0, 0)
    _check(lib.mx_clip_count(_ptr(x), _DTYPE[x.dtype], R, C, x.stride(0), ctypes.byref(cfg), _ELEM[elem][0],
                             _ptr(out), _stream(x)))
    return out


def quantize_gather(x, rows, rounding="rne", rht_mask=None, seed=0, offset=0, out=None, scale_mode="floor"):
    """Quantize the rows x[rows[i]] of a 2-D bf16/fp32 CUDA tensor, 1-D blocks
    along the last dim (see mx_quantize_gather in include/mx.h).  `rows` is an
    int32 CUDA tensor; indices outside [0, x.shape[0]) give NaN blocks."""
    lib = load_library()
    if x.dim() != 2 or x.dtype not in _DTYPE or not x.is_cuda:
        raise ValueError("quantize_gather expects a 2-D bf16/float32 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("quantize_gather expects a row-major tensor (stride(1) == 1)")
    if rows.dtype != torch.int32 or rows.dim() != 1 or not rows.is_cuda or not rows.is_contiguous():
        raise ValueError("quantize_gather expects rows as a contiguous 1-D int32 CUDA tensor")
    R, C = x.shape
    n = rows.shape[0]
    if out is None:
        out = empty_mx(n, C, "1d", x.device)
    cfg = QuantCfgC(_AXIS["last"], _BLOCK["1d"], _ROUND[rounding], int(rht_mask is not None),
                    (rht_mask or 0) & 0xFFFFFFFF, _SCALE[scale_mode], seed & (2**64 - 1),
                    offset & (2**64 - 1))
    ot = out.c_struct()
    _check(lib.mx_quantize_gather(_ptr(x), _DTYPE[x.dtype], R, C, x.stride(0), _ptr(rows), n,
                                  ctypes.byref(cfg), ctypes.byref(ot), _stream(x)))
    return out


def quantize_scatter(x, dest, k, rows_out=None, rht_mask=None, out=None, scale_mode="floor"):
    """Quantize each row of a 2-D bf16/fp32 CUDA tensor once (1-D blocks along
    the last dim, RNE) and store it to its k destination rows dest[t*k + j]
    (see mx_quantize_scatter).  `dest` is an int32 CUDA tensor of x.shape[0]*k
    entries; out (or a new [rows_out, C] operand) receives the rows."""
    lib = load_library()
    if x.dim() != 2 or x.dtype not in _DTYPE or not x.is_cuda:
        raise ValueError("quantize_scatter expects a 2-D bf16/float32 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("quantize_scatter expects a row-major tensor (stride(1) == 1)")
    R, C = x.shape
    if dest.dtype != torch.int32 or not dest.is_cuda or not dest.is_contiguous() or dest.numel() != R * k:
        raise ValueError("quantize_scatter expects dest as a contiguous int32 CUDA tensor of R*k entries")
    if out is None:
        out = empty_mx(R * k if rows_out is None else rows_out, C, "1d", x.device)
    cfg = QuantCfgC(_AXIS["last"], _BLOCK["1d"], _ROUND["rne"], int(rht_mask is not None),
                    (rht_mask or 0) & 0xFFFFFFFF, _SCALE[scale_mode], 0, 0)
    ot = out.c_struct()
    _check(lib.mx_quantize_scatter(_ptr(x), _DTYPE[x.dtype], R, C, x.stride(0), _ptr(dest), k,
                                   ctypes.byref(cfg), ctypes.byref(ot), _stream(x)))
    return out


def dequantize(q, dtype=torch.float32, inverse_rht_mask=None, out=None):
    """Decode an MX operand to a [rows, K] tensor (see mx_dequantize)."""
    lib = load_library()
    if out is None:
        out = torch.empty((q.rows, q.K), dtype=dtype, device=q.codes.device)
    qt = q.c_struct()
    _check(lib.mx_dequantize(ctypes.byref(qt), int(inverse_rht_mask is not None),
                             (inverse_rht_mask or 0) & 0xFFFFFFFF, _ptr(out), _DTYPE[out.dtype],
                             out.stride(0), _stream(out)))
    return out


def transpose(q, out=None):
    """Exact transpose of an operand with 2-D (32x32) blocks: [R, C] -> [C, R]
    (see mx_transpose)."""
    lib = load_library()
    if out is None:
        out = empty_mx(q.K, q.rows, "2d", device=q.codes.device, elem=q.elem)
    it, ot = q.c_struct(), out.c_struct()
    _check(lib.mx_transpose(ctypes.byref(it), ctypes.byref(ot), _stream(q.codes)))
    return out


_WORKSPACES = {}


def gemm_workspace(M, N, K, device="cuda"):
    """A workspace for mx_gemm of an M x N x K problem (None if it needs none):
    one zero-filled buffer per device, grown on demand and reused (every call
    leaves it fit for the next, see mx_gemm_workspace_size).  Calls that share
    it must not overlap, so callers on several streams pass their own."""
    n = load_library().mx_gemm_workspace_size(M, N, K)
    if not n:
        return None
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < n:
        ws = torch.zeros(n, dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    return ws


def gemm(a, b, out_dtype=torch.float32, out=None, workspace=None):
    """C = A * B^T for MX operands A [M, K], B [N, K] (see mx_gemm).  Shapes
    that mx_gemm splits along K use `workspace` (a zero-filled uint8 CUDA
    tensor of at least mx_gemm_workspace_size bytes) or the per-device one of
    gemm_workspace."""
    lib = load_library()
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=out_dtype, device=a.codes.device)
    ws = lib.mx_gemm_workspace_size(a.rows, b.rows, a.K)
    if ws and workspace is None:
        workspace = gemm_workspace(a.rows, b.rows, a.K, a.codes.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    at, bt = a.c_struct(), b.c_struct()
    _check(lib.mx_gemm(ctypes.byref(at), ctypes.byref(bt), _ptr(out), _DTYPE[out.dtype],
                       out.stride(0), _ptr(workspace), nbytes, _stream(out)))
    return out


def gemm_noalloc(a, b, out_dtype=torch.float32, out=None):
    """C = A * B^T through mx_gemm_noalloc: the library's own split-K scratch,
    no workspace argument (for callers that cannot allocate; the output is
    still the caller's)."""
    lib = load_library()
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=out_dtype, device=a.codes.device)
    at, bt = a.c_struct(), b.c_struct()
    _check(lib.mx_gemm_noalloc(ctypes.byref(at), ctypes.byref(bt), _ptr(out), _DTYPE[out.dtype], out.stride(0),
                               _stream(out)))
    return out


def gemm_fused_quant_a(a, b, out_dtype=torch.float32, out=None, rht_mask=None, scale_mode="floor"):
    """C = Q(A) * B^T with A a 2-D bf16 CUDA tensor [M, K] quantized to MXFP4
    inside the GEMM's operand load (RNE, 1-D blocks along K, optional
    transform; see mx_gemm_fused_quant_a) and B an MXFP4 operand [N, K]."""
    lib = load_library()
    if a.dim() != 2 or a.dtype not in _DTYPE or not a.is_cuda or a.stride(1) != 1:
        raise ValueError("gemm_fused_quant_a expects a row-major 2-D bf16 CUDA tensor")
    M, K = a.shape
    if out is None:
        out = torch.empty((M, b.rows), dtype=out_dtype, device=a.device)
    cfg = QuantCfgC(_AXIS["last"], _BLOCK["1d"], _ROUND["rne"], int(rht_mask is not None),
                    (rht_mask or 0) & 0xFFFFFFFF, _SCALE[scale_mode], 0, 0)
    bt = b.c_struct()
    _check(lib.mx_gemm_fused_quant_a(_ptr(a), _DTYPE[a.dtype], M, K, a.stride(0), ctypes.byref(cfg), ctypes.byref(bt),
                                     _ptr(out), _DTYPE[out.dtype], out.stride(0), _stream(out)))
    return out


def gemm_quantize(a, b, scale_mode="floor", out=None):
    """A * B^T quantized along N into an MXFP4 operand [M, N] (1-D blocks, RNE)
    in the GEMM epilogue (see mx_gemm_quantize)."""
    lib = load_library()
    if out is None:
        out = empty_mx(a.rows, b.rows, device=a.codes.device)
    at, bt, ot = a.c_struct(), b.c_struct(), out.c_struct()
    _check(lib.mx_gemm_quantize(ctypes.byref(at), ctypes.byref(bt), _SCALE[scale_mode], ctypes.byref(ot),
                                _stream(out.codes)))
    return out


def grouped_gemm(a, offsets, b, out_dtype=torch.bfloat16, out=None):
    """MoE grouped GEMM (see mx_grouped_gemm).

    a: MXTensor [M, K] with rows grouped by expert; offsets: int32 CUDA tensor
    [E+1]; b: MXTensor whose codes are [E, N, K/2] and scales [E, N/32, K/32]
    (2-D) or [E, N, K/32] (1-D)."""
    lib = load_library()
    E = b.codes.shape[0]
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.numel() != E + 1:
        raise ValueError("offsets must be an int32 CUDA tensor with E+1 entries")
    N = b.codes.shape[1]
    if out is None:
        out = torch.empty((a.rows, N), dtype=out_dtype, device=a.codes.device)
    b0 = MxTensorC(b.codes.data_ptr(), b.scales.data_ptr(), N, b.K, b.codes.stride(1),
                   b.scales.stride(1), _BLOCK[b.block], _ELEM[b.elem][0])
    at = a.c_struct()
    _check(lib.mx_grouped_gemm(ctypes.byref(at), _ptr(offsets), E, ctypes.byref(b0),
                               b.codes.stride(0), b.scales.stride(0), _ptr(out),
                               _DTYPE[out.dtype], out.stride(0), _stream(out)))
    return out


def grouped_gemm_quantize(a, offsets, b, scale_mode="floor", out=None):
    """The grouped product quantized along N into an MXFP4 operand [M, N] in
    the GEMM epilogue (see mx_grouped_gemm_quantize); arguments as
    grouped_gemm."""
    lib = load_library()
    E = b.codes.shape[0]
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.numel() != E + 1:
        raise ValueError("offsets must be an int32 CUDA tensor with E+1 entries")
    N = b.codes.shape[1]
    if out is None:
        out = empty_mx(a.rows, N, device=a.codes.device)
    b0 = MxTensorC(b.codes.data_ptr(), b.scales.data_ptr(), N, b.K, b.codes.stride(1),
                   b.scales.stride(1), _BLOCK[b.block], _ELEM[b.elem][0])
    at, ot = a.c_struct(), out.c_struct()
    _check(lib.mx_grouped_gemm_quantize(ctypes.byref(at), _ptr(offsets), E, ctypes.byref(b0), b.codes.stride(0),
                                        b.scales.stride(0), _SCALE[scale_mode], ctypes.byref(ot),
                                        _stream(out.codes)))
    return out


def version():
    return load_library().mx_version().decode()
