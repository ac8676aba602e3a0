"""ctypes binding of libsattn (include/sattn.h) with the same entry-point names, plus torch marshalling.

Every step of the computation runs in the HIP kernels of libsattn.so; this module only turns torch tensors
into pointers, sizes and the current HIP stream, and raises ``SattnError`` for a non-OK status.  There is
no CPU fallback: if the library is missing, importing the entry points fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsattn.so")

SATTN_OK = 0
SATTN_ERR_INVALID_ARG = 1
SATTN_ERR_UNSUPPORTED = 2
SATTN_ERR_WORKSPACE = 3
SATTN_ERR_HIP = 4

SATTN_MODE_BF16 = 0
SATTN_MODE_I8_BF16 = 1
SATTN_MODE_I8_FP8 = 2

SATTN_LINEAR_BLK = 128
SATTN_LINEAR_W8A8 = 0
SATTN_LINEAR_W8A16 = 1


class SattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sattn_status_string(status)} (status {status})")


class sattn_tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int),
                ("d", ctypes.c_int), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_n", ctypes.c_int64)]


class sattn_quant(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("Nq", ctypes.c_int), ("Nkv", ctypes.c_int),
                ("d", ctypes.c_int), ("blk_q", ctypes.c_int), ("blk_k", ctypes.c_int), ("mode", ctypes.c_int),
                ("q_codes", ctypes.c_void_p), ("q_scales", ctypes.c_void_p), ("k_codes", ctypes.c_void_p),
                ("k_scales", ctypes.c_void_p), ("k_mean", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("v_t", ctypes.c_void_p)]


_lib = None

# (name, restype, argtypes) for every symbol declared in include/sattn.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_TP = ctypes.POINTER(sattn_tensor)
_QP = ctypes.POINTER(sattn_quant)
SYMBOLS = [
    ("sattn_status_string", ctypes.c_char_p, [_I]),
    ("sattn_kv_tile", _I, [_I, _I]),
    ("sattn_quant_bytes", _SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    ("sattn_quant_layout", _I, [_I, _I, _I, _I, _I, _I, _I, _I, _P, _QP]),
    ("sattn_workspace_bytes", _SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    ("sattn_quantize_scratch_bytes", _SZ, [_I, _I, _I, _I, _I]),
    ("sattn_quantize", _I, [_TP, _TP, _TP, _I, _QP, _P, _SZ, _P]),
    ("sattn_fwd_quantized", _I, [_TP, _TP, _QP, _TP, ctypes.c_float, _I, _P]),
    ("sattn_fwd", _I, [_TP, _TP, _TP, _TP, ctypes.c_float, _I, _I, _I, _P, _SZ, _P]),
    ("sattn_fwd_noalloc", _I, [_TP, _TP, _TP, _TP, ctypes.c_float, _I, _I, _I, _P]),
    ("sattn_cross_fwd", _I, [_TP, _TP, _TP, _TP, ctypes.c_float, _I, _P, _SZ, _P]),
    ("sattn_fwd_block_sparse", _I, [_TP, _TP, _TP, _TP, _P, ctypes.c_float, _I, _I, _I, _P, _SZ, _P]),
    ("sattn_error_stats_workspace_bytes", _SZ, [_I, _I, _I]),
    ("sattn_error_stats", _I, [_TP, _TP, _P, _P, _SZ, _P]),
    ("sattn_debug_qk_int32", _I, [_QP, _I, _I, _I, _I, _I, _I, _P, _P]),
    ("sattn_quantize_blocks", _I, [_P, _I, _I, ctypes.c_int64, _P, _P, _P]),
    ("sattn_linear_workspace_bytes", _SZ, [_I, _I, _I, _I]),
    ("sattn_linear_quantized", _I, [_P, _P, _P, _P, _P, _P, ctypes.c_int64, _I, _I, _I, _P]),
    ("sattn_linear", _I, [_P, ctypes.c_int64, _P, _P, _P, _P, ctypes.c_int64, _I, _I, _I, _I, _P, _SZ, _P]),
]


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quantized_attention_05_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SYMBOLS:
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


# ------------------------------------------------------------------------------------- raw entry points
def sattn_status_string(st: int) -> str:
    return lib().sattn_status_string(int(st)).decode()


def sattn_kv_tile(d: int, mode: int) -> int:
    return int(lib().sattn_kv_tile(d, mode))


def sattn_quant_bytes(B, H, Nq, Nkv, d, blk_q, blk_k, mode) -> int:
    return int(lib().sattn_quant_bytes(B, H, Nq, Nkv, d, blk_q, blk_k, mode))


def sattn_workspace_bytes(B, H, Nq, Nkv, d, blk_q, blk_k, mode) -> int:
    return int(lib().sattn_workspace_bytes(B, H, Nq, Nkv, d, blk_q, blk_k, mode))


def sattn_quantize_scratch_bytes(B, H, Nkv, d, mode) -> int:
    return int(lib().sattn_quantize_scratch_bytes(B, H, Nkv, d, mode))


def _check(st: int, where: str):
    if st != SATTN_OK:
        raise SattnError(st, where)


def sattn_quant_layout(B, H, Nq, Nkv, d, blk_q, blk_k, mode, base: int) -> sattn_quant:
    out = sattn_quant()
    _check(lib().sattn_quant_layout(B, H, Nq, Nkv, d, blk_q, blk_k, mode, ctypes.c_void_p(base), ctypes.byref(out)),
           "sattn_quant_layout")
    return out


def sattn_quantize(q, k, v, mode, out: sattn_quant, scratch: int, scratch_bytes: int, stream: int):
    _check(lib().sattn_quantize(_ref(q), _ref(k), _ref(v), mode, ctypes.byref(out), ctypes.c_void_p(scratch),
                                scratch_bytes, ctypes.c_void_p(stream)), "sattn_quantize")


def sattn_fwd_quantized(q, k, qk: sattn_quant, o, sm_scale, mode, stream: int):
    _check(lib().sattn_fwd_quantized(_ref(q), _ref(k), ctypes.byref(qk), _ref(o), float(sm_scale), mode,
                                     ctypes.c_void_p(stream)), "sattn_fwd_quantized")


def sattn_fwd(q, k, v, o, sm_scale, mode, blk_q, blk_k, ws: int, ws_bytes: int, stream: int):
    _check(lib().sattn_fwd(_ref(q), _ref(k), _ref(v), _ref(o), float(sm_scale), mode, blk_q, blk_k,
                           ctypes.c_void_p(ws), ws_bytes, ctypes.c_void_p(stream)), "sattn_fwd")


def sattn_fwd_noalloc(q, k, v, o, sm_scale, mode, blk_q, blk_k, stream: int):
    _check(lib().sattn_fwd_noalloc(_ref(q), _ref(k), _ref(v), _ref(o), float(sm_scale), mode, blk_q, blk_k,
                                   ctypes.c_void_p(stream)), "sattn_fwd_noalloc")


def sattn_cross_fwd(q, k, v, o, sm_scale, mode, ws: int, ws_bytes: int, stream: int):
    _check(lib().sattn_cross_fwd(_ref(q), _ref(k), _ref(v), _ref(o), float(sm_scale), mode, ctypes.c_void_p(ws),
                                 ws_bytes, ctypes.c_void_p(stream)), "sattn_cross_fwd")


def sattn_fwd_block_sparse(q, k, v, o, block_mask: int, sm_scale, mode, blk_q, blk_k, ws: int, ws_bytes: int,
                           stream: int):
    _check(lib().sattn_fwd_block_sparse(_ref(q), _ref(k), _ref(v), _ref(o), ctypes.c_void_p(block_mask),
                                        float(sm_scale), mode, blk_q, blk_k, ctypes.c_void_p(ws), ws_bytes,
                                        ctypes.c_void_p(stream)), "sattn_fwd_block_sparse")


def sattn_error_stats_workspace_bytes(B, H, N) -> int:
    return lib().sattn_error_stats_workspace_bytes(B, H, N)


def sattn_error_stats(a, ref, out: int, ws: int, ws_bytes: int, stream: int):
    _check(lib().sattn_error_stats(_ref(a), _ref(ref), ctypes.c_void_p(out), ctypes.c_void_p(ws), ws_bytes,
                                   ctypes.c_void_p(stream)), "sattn_error_stats")


def sattn_debug_qk_int32(qk: sattn_quant, b, h, q0, nq, k0, nk, out: int, stream: int):
    _check(lib().sattn_debug_qk_int32(ctypes.byref(qk), b, h, q0, nq, k0, nk, ctypes.c_void_p(out),
                                      ctypes.c_void_p(stream)), "sattn_debug_qk_int32")


def _ref(t):
    return None if t is None else ctypes.byref(t)


# ------------------------------------------------------------------------------------- torch marshalling
def tensor_desc(t: torch.Tensor | None) -> sattn_tensor | None:
    """sattn_tensor for a 4-D bf16 GPU tensor indexed [B, H, N, d] (any strides with d contiguous)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("expected a GPU tensor: the kernels dereference its pointer on the device")
    if t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a 4-D bf16 tensor [B, H, N, d] with contiguous channels")
    B, H, N, d = t.shape
    return sattn_tensor(t.data_ptr(), B, H, N, d, t.stride(0), t.stride(1), t.stride(2))


def _same_device(name: str, *tensors) -> torch.device:
    """The one GPU every given tensor lives on (None entries are skipped); ValueError before any C call otherwise."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name}: every tensor must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: tensors on {dev} and {t.device}; all must share one GPU")
    if dev is None:
        raise ValueError(f"{name}: no GPU tensor given")
    return dev


def _workspace(name: str, ws, need: int, dev: torch.device) -> torch.Tensor:
    """The caller's workspace (a uint8 GPU tensor on `dev`, contiguous, at least `need` bytes) or a new one."""
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != dev:
        raise ValueError(f"{name}: the workspace must be a GPU tensor on {dev}")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError(f"{name}: the workspace must be a contiguous uint8 tensor")
    return ws


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _resolve(sm_scale, d):
    return 0.0 if sm_scale is None else float(sm_scale)


def fwd(q, k, v, mode=SATTN_MODE_I8_FP8, sm_scale=None, blk_q=128, blk_k=64, out=None, workspace=None):
    """Self-attention through sattn_fwd.  q, k, v: [B, H, N, d] bf16 on the GPU.  Returns O like q."""
    dev = _same_device("fwd", q, k, v, out)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    o = torch.empty_like(q) if out is None else out
    need = sattn_workspace_bytes(B, H, Nq, Nkv, d, blk_q, blk_k, mode)
    if need == 0:
        raise SattnError(SATTN_ERR_UNSUPPORTED, "sattn_workspace_bytes")
    ws = _workspace("fwd", workspace, need, dev)
    sattn_fwd(tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o), _resolve(sm_scale, d), mode, blk_q, blk_k,
              ws.data_ptr(), ws.numel(), _stream())
    return o


NOALLOC_SCRATCH_BYTES = 256 << 20  # SATTN_NOALLOC_SCRATCH_BYTES


def fwd_noalloc(q, k, v, out, mode=SATTN_MODE_I8_FP8, sm_scale=None, blk_q=128, blk_k=64):
    """Self-attention through sattn_fwd_noalloc: the workspace is the library's own per-GPU array, so the call allocates
    nothing; the caller passes the output `out` ([B, H, Nq, d] bf16 on the GPU of q)."""
    _same_device("fwd_noalloc", q, k, v, out)
    sattn_fwd_noalloc(tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(out), _resolve(sm_scale, q.shape[3]),
                      mode, blk_q, blk_k, _stream())
    return out


MASK_QBLK = 128  # query rows per block-sparse mask row (SATTN_MASK_QBLK)
MASK_KBLK = 64   # keys per block-sparse mask column (SATTN_MASK_KBLK)


def mask_shape(B, H, Nq, Nkv):
    """Shape of the block-sparse mask of sattn_fwd_block_sparse: [B, H, ceil(Nq/128), ceil(Nkv/64)]."""
    return (B, H, -(-Nq // MASK_QBLK), -(-Nkv // MASK_KBLK))


def fwd_block_sparse(q, k, v, mask, mode=SATTN_MODE_I8_FP8, sm_scale=None, blk_q=128, blk_k=64, out=None,
                     workspace=None):
    """Block-sparse self-attention through sattn_fwd_block_sparse.  mask: uint8 (nonzero = keep) on the GPU, shaped
    mask_shape(B, H, Nq, Nkv), contiguous.  Returns O like q."""
    dev = _same_device("fwd_block_sparse", q, k, v, mask, out)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if tuple(mask.shape) != mask_shape(B, H, Nq, Nkv) or mask.dtype != torch.uint8 or not mask.is_contiguous():
        raise SattnError(SATTN_ERR_INVALID_ARG, "fwd_block_sparse: mask shape/dtype/layout")
    o = torch.empty_like(q) if out is None else out
    need = sattn_workspace_bytes(B, H, Nq, Nkv, d, blk_q, blk_k, mode)
    if need == 0:
        raise SattnError(SATTN_ERR_UNSUPPORTED, "sattn_workspace_bytes")
    ws = _workspace("fwd_block_sparse", workspace, need, dev)
    sattn_fwd_block_sparse(tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o), mask.data_ptr(),
                           _resolve(sm_scale, d), mode, blk_q, blk_k, ws.data_ptr(), ws.numel(), _stream())
    return o


def cross_fwd(q, k, v, mode=SATTN_MODE_BF16, sm_scale=None, out=None, workspace=None):
    """Cross-attention through sattn_cross_fwd (short key sequence).  Returns O like q."""
    dev = _same_device("cross_fwd", q, k, v, out)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    o = torch.empty_like(q) if out is None else out
    need = sattn_workspace_bytes(B, H, Nq, Nkv, d, 128, 64, mode)
    if need == 0:
        raise SattnError(SATTN_ERR_UNSUPPORTED, "sattn_workspace_bytes")
    ws = _workspace("cross_fwd", workspace, need, dev)
    sattn_cross_fwd(tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o), _resolve(sm_scale, d), mode,
                    ws.data_ptr(), ws.numel(), _stream())
    return o


def error_stats(a, ref, workspace=None):
    """Per-head fp64 sums [sum (a-ref)^2, sum ref^2, sum a*ref, sum a^2] of two [B, H, N, d] bf16 GPU tensors
    through sattn_error_stats.  Returns a [B, H, 4] float64 GPU tensor."""
    dev = _same_device("error_stats", a, ref)
    B, H, N = a.shape[0], a.shape[1], a.shape[2]
    ws = _workspace("error_stats", workspace, sattn_error_stats_workspace_bytes(B, H, N), dev)
    out = torch.empty((B, H, 4), dtype=torch.float64, device=dev)
    sattn_error_stats(tensor_desc(a), tensor_desc(ref), out.data_ptr(), ws.data_ptr(), ws.numel(), _stream())
    return out


class Quantized:
    """Quantized operands in one device buffer, with torch views of each array (see sattn_quant)."""

    def __init__(self, B, H, Nq, Nkv, d, blk_q, mode, device, blk_k=64):
        if torch.device(device).type != "cuda":
            raise ValueError("Quantized: the code buffer must live on a GPU")
        self.shape = (B, H, Nq, Nkv, d, blk_q, blk_k, mode)
        nbytes = sattn_quant_bytes(B, H, Nq, Nkv, d, blk_q, blk_k, mode)
        if nbytes == 0:
            raise SattnError(SATTN_ERR_UNSUPPORTED, "sattn_quant_bytes")
        self.buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
        base = (self.buf.data_ptr() + 255) // 256 * 256
        self.desc = sattn_quant_layout(B, H, Nq, Nkv, d, blk_q, blk_k, mode, base)
        self._base = base
        nqb, nkb = -(-Nq // blk_q), -(-Nkv // 64)
        self.nqb, self.nkb = nqb, nkb
        self.mode = mode

        def view(ptr, numel, dtype, shape):
            if not ptr:
                return None
            off = ptr - self.buf.data_ptr()
            nb = numel * torch.tensor([], dtype=dtype).element_size()
            return self.buf[off:off + nb].view(dtype).view(shape)

        D = self.desc
        self.q_codes = view(D.q_codes, B * H * nqb * blk_q * d, torch.int8, (B, H, nqb * blk_q, d))
        self.q_scales = view(D.q_scales, B * H * nqb, torch.float32, (B, H, nqb))
        self.k_codes = view(D.k_codes, B * H * nkb * 64 * d, torch.int8, (B, H, nkb * 64, d))
        self.k_scales = view(D.k_scales, B * H * nkb, torch.float32, (B, H, nkb))
        self.k_mean = view(D.k_mean, B * H * d, torch.float32, (B, H, d))
        self.v_codes = view(D.v_codes, B * H * nkb * d * 64, torch.uint8, (B, H, nkb, d, 64))
        self.v_scales = view(D.v_scales, B * H * d, torch.float32, (B, H, d))
        self.v_t = view(D.v_t, B * H * nkb * d * 64, torch.int16, (B, H, nkb, d, 64))


def quantize(q, k, v, mode=SATTN_MODE_I8_FP8, blk_q=128, quant: Quantized | None = None):
    """Run sattn_quantize; returns a ``Quantized`` holding the codes/scales (device tensors)."""
    dev = _same_device("quantize", q, k, v, None if quant is None else quant.buf)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    qz = quant if quant is not None else Quantized(B, H, Nq, Nkv, d, blk_q, mode, dev)
    sb = sattn_quantize_scratch_bytes(B, H, Nkv, d, mode)
    scratch = torch.empty(max(sb, 1), dtype=torch.uint8, device=dev)
    sattn_quantize(tensor_desc(q), tensor_desc(k), tensor_desc(v), mode, qz.desc, scratch.data_ptr(), sb, _stream())
    qz._scratch = scratch  # keep alive until the stream has used it
    return qz


def fwd_quantized(qz: Quantized, q=None, k=None, sm_scale=None, out=None):
    """Attention on prepared operands through sattn_fwd_quantized."""
    dev = _same_device("fwd_quantized", qz.buf, q, k, out)
    B, H, Nq, Nkv, d, blk_q, blk_k, mode = qz.shape
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=dev)
    sattn_fwd_quantized(tensor_desc(q), tensor_desc(k), qz.desc, tensor_desc(out), _resolve(sm_scale, d), mode,
                        _stream())
    return out


def debug_qk_int32(qz: Quantized, b, h, q0, nq, k0, nk):
    out = torch.empty((nq, nk), dtype=torch.int32, device=qz.buf.device)
    sattn_debug_qk_int32(qz.desc, b, h, q0, nq, k0, nk, out.data_ptr(), _stream())
    return out


# ---------------------------------------------------------------- quantized linear layer
def sattn_quantize_blocks(x: int, rows, cols, ld, codes: int, scales: int, stream: int):
    _check(lib().sattn_quantize_blocks(_P(x), rows, cols, ld, _P(codes), _P(scales), _P(stream)),
           "sattn_quantize_blocks")


def sattn_linear_workspace_bytes(M, N, K, mode) -> int:
    return int(lib().sattn_linear_workspace_bytes(M, N, K, mode))


def sattn_linear_quantized(xq: int, sx: int, wq: int, sw: int, bias: int | None, y: int, ldy, M, N, K, stream: int):
    _check(lib().sattn_linear_quantized(_P(xq), _P(sx), _P(wq), _P(sw), _P(bias), _P(y), ldy, M, N, K, _P(stream)),
           "sattn_linear_quantized")


def sattn_linear(x: int, ldx, wq: int, sw: int, bias: int | None, y: int, ldy, M, N, K, mode, ws: int, ws_bytes: int,
                 stream: int):
    _check(lib().sattn_linear(_P(x), ldx, _P(wq), _P(sw), _P(bias), _P(y), ldy, M, N, K, mode, _P(ws), ws_bytes,
                              _P(stream)), "sattn_linear")


def _rows(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    """A 2-D view [rows, cols] with unit column stride on the GPU (leading dimensions are flattened)."""
    if t.dtype != dtype or not t.is_cuda:
        raise ValueError(f"{name}: expected a {dtype} CUDA tensor, got {t.dtype} on {t.device}")
    t2 = t.view(-1, t.shape[-1]) if t.dim() != 2 else t  # a view, never a copy (outputs are written through it)
    if t2.stride(1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return t2


def quantize_blocks(x: torch.Tensor):
    """Per-block INT8 of a bf16 matrix (e.g. a linear weight [N, K]) in 128 x 128 blocks: (codes int8 [rows, cols],
    scales float32 [ceil(rows/128), cols/128])."""
    x2 = _rows(x, torch.bfloat16, "x")
    rows, cols = x2.shape
    codes = torch.empty((rows, cols), dtype=torch.int8, device=x2.device)
    nbc = cols // SATTN_LINEAR_BLK if cols % SATTN_LINEAR_BLK == 0 else 1  # (other widths are refused by the call)
    scales = torch.empty((-(-rows // SATTN_LINEAR_BLK), nbc), dtype=torch.float32, device=x2.device)
    sattn_quantize_blocks(x2.data_ptr(), rows, cols, x2.stride(0), codes.data_ptr(), scales.data_ptr(), _stream())
    return codes, scales


def _linear_out(x_rows: int, N: int, out, device):
    if out is None:
        return torch.empty((x_rows, N), dtype=torch.bfloat16, device=device)
    o2 = _rows(out, torch.bfloat16, "out")
    if o2.shape != (x_rows, N):
        raise ValueError(f"out: expected {(x_rows, N)} rows x columns, got {tuple(o2.shape)}")
    return o2


def linear_quantized(xq: torch.Tensor, sx: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor, bias=None, out=None):
    """W8A8 linear on prepared codes (sattn_linear_quantized): y [M, N] bf16."""
    xq2, wq2 = _rows(xq, torch.int8, "xq"), _rows(wq, torch.int8, "wq")
    M, K = xq2.shape
    N = wq2.shape[0]
    if wq2.shape[1] != K or not xq2.is_contiguous() or not wq2.is_contiguous():
        raise ValueError("xq [M, K] and wq [N, K] must be dense with the same K")
    for t, name in ((sx, "sx"), (sw, "sw")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name}: expected a dense float32 CUDA tensor")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous()):
        raise ValueError("bias: expected a dense bf16 tensor of N elements")
    y = _linear_out(M, N, out, xq2.device)
    sattn_linear_quantized(xq2.data_ptr(), sx.data_ptr(), wq2.data_ptr(), sw.data_ptr(),
                           None if bias is None else bias.data_ptr(), y.data_ptr(), y.stride(0), M, N, K, _stream())
    return y


def linear(x: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor, bias=None, mode=SATTN_LINEAR_W8A8, out=None,
           workspace=None):
    """The quantized linear layer y = x W^T + bias (sattn_linear) for bf16 x [..., K] and a weight prepared by
    quantize_blocks; returns y [..., N] bf16.  mode: SATTN_LINEAR_W8A8 or SATTN_LINEAR_W8A16."""
    x2 = _rows(x, torch.bfloat16, "x")
    wq2 = _rows(wq, torch.int8, "wq")
    M, K = x2.shape
    N = wq2.shape[0]
    if wq2.shape[1] != K or not wq2.is_contiguous():
        raise ValueError("wq must be dense [N, K] with the K of x")
    if sw.dtype != torch.float32 or not sw.is_cuda or not sw.is_contiguous():
        raise ValueError("sw: expected a dense float32 CUDA tensor")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous()):
        raise ValueError("bias: expected a dense bf16 tensor of N elements")
    y = _linear_out(M, N, out, x2.device)
    need = sattn_linear_workspace_bytes(M, N, K, mode)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x2.device)
    sattn_linear(x2.data_ptr(), x2.stride(0), wq2.data_ptr(), sw.data_ptr(), None if bias is None else bias.data_ptr(),
                 y.data_ptr(), y.stride(0), M, N, K, mode, workspace.data_ptr(), workspace.numel(), _stream())
    return y.view(*x.shape[:-1], N) if x.dim() != 2 else y
