"""CPU oracle for SageAttention-style quantized attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import this
package.  The GPU library (``quantized_attention_05_amd``) never imports it, and the two share no code:
the arithmetic lives in ``sattn_oracle.c`` (plain C loops, fp32 for every step that produces a code,
int64 scores, fp64 elsewhere); this module only marshals numpy arrays into it.

bf16 tensors are passed as their raw 16-bit patterns (``numpy.uint16``); E4M3 codes as ``numpy.uint8``.
Every array handed to the C side is one (batch, head) slice, dense row-major ``[tokens, d]``.

Functions mirror the steps of the method:

* ``k_mean``      per-channel mean of K (two-level sequential fp32 order)
* ``quant_q``     per-block INT8 quantization of Q with the zero guard
* ``quant_k``     smoothing (K - mean) followed by per-block INT8 quantization
* ``quant_v``     per-channel E4M3 quantization of V with the zero guard
* ``qk_int``      exact integer scores
* ``attn_emulate``  tile-faithful replay of dequant + online softmax + P*V + epilogue (modes 0/1/2)
* ``attn_ref_fp64`` exact attention in fp64 (what the quantized modes approximate)
* ``quant_blocks``, ``linear_w8a8``, ``linear_w8a16``  the 128 x 128 per-block quantized linear layer
  (``linear_oracle.c``)

Parity pins for all of them are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "sattn_oracle.c"), os.path.join(_HERE, "linear_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "libsattn_oracle.so")

MODE_BF16 = 0
MODE_I8_BF16 = 1
MODE_I8_FP8 = 2

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile ``sattn_oracle.c`` and ``linear_oracle.c`` into ``libsattn_oracle.so`` next to them (plain gcc, no
    HIP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_double
        L.orc_bf16_from_f32.argtypes, L.orc_bf16_from_f32.restype = [f32], ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes, L.orc_bf16_to_f32.restype = [ctypes.c_uint16], f32
        L.orc_e4m3_decode.argtypes, L.orc_e4m3_decode.restype = [ctypes.c_uint8], f32
        L.orc_e4m3_encode.argtypes, L.orc_e4m3_encode.restype = [f32], ctypes.c_uint8
        L.orc_k_mean.argtypes, L.orc_k_mean.restype = [P, i32, i32, i64, P], None
        L.orc_quant_q.argtypes, L.orc_quant_q.restype = [P, i32, i32, i64, i32, P, P], None
        L.orc_quant_k.argtypes, L.orc_quant_k.restype = [P, i32, i32, i64, P, i32, P, P], None
        L.orc_quant_v.argtypes, L.orc_quant_v.restype = [P, i32, i32, i64, P, P], None
        L.orc_qk_int.argtypes, L.orc_qk_int.restype = [P, i32, P, i32, i32, P], None
        L.orc_attn_emulate.argtypes = [i32, i32, i32, i32, i32, i32, f32, P, P, P, P, P, P, P, P, P, P, i32, P, P]
        L.orc_attn_emulate.restype = None
        L.orc_attn_ref_fp64.argtypes = [i32, i32, f64, P, P, P, P, i32, P]
        L.orc_attn_ref_fp64.restype = None
        L.orc_attn_emulate_masked.argtypes = [i32, i32, i32, i32, i32, i32, f32, P, P, P, P, P, P, P, P, P, P, i32,
                                              P, i32, P, P]
        L.orc_attn_emulate_masked.restype = None
        L.orc_attn_ref_fp64_masked.argtypes = [i32, i32, f64, P, P, P, P, i32, P, i32, P]
        L.orc_attn_ref_fp64_masked.restype = None
        L.orc_max_threads.argtypes, L.orc_max_threads.restype = [], i32
        L.orc_quant_blocks.argtypes, L.orc_quant_blocks.restype = [P, i32, i32, i64, i32, i32, P, P], None
        L.orc_linear_w8a8.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P, P]
        L.orc_linear_w8a8.restype = None
        L.orc_linear_w8a16.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P]
        L.orc_linear_w8a16.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dense(a: np.ndarray, dtype) -> np.ndarray:
    assert a.dtype == dtype, (a.dtype, dtype)
    return np.ascontiguousarray(a)


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- number formats (scalar, vectorised)
def bf16_from_f32(x) -> np.ndarray:
    L = lib()
    x = np.asarray(x, dtype=np.float32)
    return np.array([L.orc_bf16_from_f32(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def bf16_to_f32(h) -> np.ndarray:
    L = lib()
    h = np.asarray(h, dtype=np.uint16)
    return np.array([L.orc_bf16_to_f32(int(v)) for v in h.ravel()], dtype=np.float32).reshape(h.shape)


def e4m3_decode(c) -> np.ndarray:
    L = lib()
    c = np.asarray(c, dtype=np.uint8)
    return np.array([L.orc_e4m3_decode(int(v)) for v in c.ravel()], dtype=np.float32).reshape(c.shape)


def e4m3_encode(x) -> np.ndarray:
    L = lib()
    x = np.asarray(x, dtype=np.float32)
    return np.array([L.orc_e4m3_encode(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


# ---------------------------------------------------------------- quantization steps (one head slice)
def k_mean(k_bf16: np.ndarray) -> np.ndarray:
    k = _dense(k_bf16, np.uint16)
    n, d = k.shape
    mu = np.empty(d, dtype=np.float32)
    lib().orc_k_mean(_ptr(k), n, d, d, _ptr(mu))
    return mu


def _nblk(n: int, blk: int) -> int:
    return (n + blk - 1) // blk


def quant_q(q_bf16: np.ndarray, blk: int):
    q = _dense(q_bf16, np.uint16)
    n, d = q.shape
    nb = _nblk(n, blk)
    codes = np.empty((nb * blk, d), dtype=np.int8)
    scales = np.empty(nb, dtype=np.float32)
    lib().orc_quant_q(_ptr(q), n, d, d, blk, _ptr(codes), _ptr(scales))
    return codes, scales


def quant_k(k_bf16: np.ndarray, blk: int, mu: np.ndarray):
    k = _dense(k_bf16, np.uint16)
    mu = _dense(mu, np.float32)
    n, d = k.shape
    nb = _nblk(n, blk)
    codes = np.empty((nb * blk, d), dtype=np.int8)
    scales = np.empty(nb, dtype=np.float32)
    lib().orc_quant_k(_ptr(k), n, d, d, _ptr(mu), blk, _ptr(codes), _ptr(scales))
    return codes, scales


def quant_v(v_bf16: np.ndarray):
    v = _dense(v_bf16, np.uint16)
    n, d = v.shape
    codes = np.empty((n, d), dtype=np.uint8)
    scales = np.empty(d, dtype=np.float32)
    lib().orc_quant_v(_ptr(v), n, d, d, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_head(q_bf16, k_bf16, v_bf16, blk_q: int, blk_k: int, mode: int) -> dict:
    """All quantization steps for one (batch, head) slice."""
    out = {}
    out["q_codes"], out["q_scales"] = quant_q(q_bf16, blk_q)
    out["k_mean"] = k_mean(k_bf16)
    out["k_codes"], out["k_scales"] = quant_k(k_bf16, blk_k, out["k_mean"])
    if mode == MODE_I8_FP8:
        out["v_codes"], out["v_scales"] = quant_v(v_bf16)
    return out


def qk_int(q_codes: np.ndarray, k_codes: np.ndarray) -> np.ndarray:
    qc = _dense(q_codes, np.int8)
    kc = _dense(k_codes, np.int8)
    assert qc.shape[1] == kc.shape[1]
    s = np.empty((qc.shape[0], kc.shape[0]), dtype=np.int64)
    lib().orc_qk_int(_ptr(qc), qc.shape[0], _ptr(kc), kc.shape[0], qc.shape[1], _ptr(s))
    return s


# ---------------------------------------------------------------- attention
MASK_KBLK = 64  # keys per block of a block-sparse mask


def _mask_arg(mask, rows, nkv: int, mask_qblk: int):
    """A [query blocks, key blocks] byte mask checked against the rows and keys it must cover."""
    m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    nkb = -(-nkv // MASK_KBLK)
    assert m.ndim == 2 and m.shape[1] == nkb, (m.shape, nkb)
    assert rows.size == 0 or m.shape[0] > int(rows.max()) // mask_qblk
    return m


def attn_emulate(mode: int, rows, *, tile: int, sm_scale: float, blk_q: int, blk_k: int, nkv: int,
                 q_bf16=None, k_bf16=None, v_bf16=None, quant: dict | None = None, want_f32: bool = False,
                 mask=None, mask_qblk: int = 128):
    """Tile-faithful replay of the quantized attention for the given query rows of one head slice.

    mode 0 needs q_bf16, k_bf16, v_bf16; mode 1 needs quant (q/k codes and scales) and v_bf16;
    mode 2 needs quant including v_codes/v_scales.  Returns bf16 bit patterns [len(rows), d]
    (and the fp32 values before the final rounding if want_f32).  With mask ([ceil(rows/mask_qblk),
    ceil(nkv/64)], nonzero = keep), only the kept key blocks of a row's query block take part.
    """
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    qb = kb = vb = qc = qs = kc = ks = vc = vs = None
    if mode == MODE_BF16:
        qb, kb, vb = _dense(q_bf16, np.uint16), _dense(k_bf16, np.uint16), _dense(v_bf16, np.uint16)
        d = qb.shape[1]
        assert kb.shape[0] >= nkv and vb.shape[0] >= nkv
    else:
        qc, qs = _dense(quant["q_codes"], np.int8), _dense(quant["q_scales"], np.float32)
        kc, ks = _dense(quant["k_codes"], np.int8), _dense(quant["k_scales"], np.float32)
        d = qc.shape[1]
        assert kc.shape[0] >= nkv
        if mode == MODE_I8_BF16:
            vb = _dense(v_bf16, np.uint16)
            assert vb.shape[0] >= nkv
        else:
            vc, vs = _dense(quant["v_codes"], np.uint8), _dense(quant["v_scales"], np.float32)
            assert vc.shape[0] >= nkv
    out = np.empty((rows.size, d), dtype=np.uint16)
    of = np.empty((rows.size, d), dtype=np.float32) if want_f32 else None
    if mask is None:
        lib().orc_attn_emulate(mode, nkv, d, blk_q, blk_k, tile, float(sm_scale), _ptr(qb), _ptr(kb), _ptr(qc),
                               _ptr(qs), _ptr(kc), _ptr(ks), _ptr(vb), _ptr(vc), _ptr(vs), _ptr(rows), rows.size,
                               _ptr(out), _ptr(of))
    else:
        m = _mask_arg(mask, rows, nkv, mask_qblk)
        lib().orc_attn_emulate_masked(mode, nkv, d, blk_q, blk_k, tile, float(sm_scale), _ptr(qb), _ptr(kb), _ptr(qc),
                                      _ptr(qs), _ptr(kc), _ptr(ks), _ptr(vb), _ptr(vc), _ptr(vs), _ptr(rows),
                                      rows.size, _ptr(m), mask_qblk, _ptr(out), _ptr(of))
    return (out, of) if want_f32 else out


def attn_ref_fp64(q_bf16, k_bf16, v_bf16, rows, sm_scale: float, mask=None, mask_qblk: int = 128) -> np.ndarray:
    """Exact attention softmax(c*q*K^T)*V in fp64 for the given rows of one head slice (with mask: over the
    keys of the kept key blocks; a row with none gives 0)."""
    qb, kb, vb = _dense(q_bf16, np.uint16), _dense(k_bf16, np.uint16), _dense(v_bf16, np.uint16)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    d = qb.shape[1]
    out = np.empty((rows.size, d), dtype=np.float64)
    if mask is None:
        lib().orc_attn_ref_fp64(kb.shape[0], d, float(sm_scale), _ptr(qb), _ptr(kb), _ptr(vb), _ptr(rows), rows.size,
                                _ptr(out))
    else:
        m = _mask_arg(mask, rows, kb.shape[0], mask_qblk)
        lib().orc_attn_ref_fp64_masked(kb.shape[0], d, float(sm_scale), _ptr(qb), _ptr(kb), _ptr(vb), _ptr(rows),
                                       rows.size, _ptr(m), mask_qblk, _ptr(out))
    return out


# ---------------------------------------------------------------- per-layer error probe
def error_stats(a_bits, r_bits) -> np.ndarray:
    """The probe's sums for one head slice, by definition, in fp64: [sum (a-r)^2, sum r^2, sum a*r, sum a^2] over all
    elements of two bf16 arrays (16-bit patterns) of equal shape."""
    a = (np.asarray(a_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = (np.asarray(r_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert a.shape == r.shape
    d = a - r
    return np.array([np.sum(d * d), np.sum(r * r), np.sum(a * r), np.sum(a * a)])


# ---------------------------------------------------------------- the quantized linear layer (linear_oracle.c)
LINEAR_BLK = 128


def quant_blocks(x_bits, blk: int = LINEAR_BLK):
    """Per-block INT8 of a bf16 matrix [rows, cols] (16-bit patterns) in blk x blk blocks: (codes int8 [rows, cols],
    scales float32 [ceil(rows/blk), ceil(cols/blk)])."""
    x = _dense(np.asarray(x_bits), np.uint16)
    rows, cols = x.shape
    codes = np.empty((rows, cols), np.int8)
    scales = np.empty((_nblk(rows, blk), _nblk(cols, blk)), np.float32)
    lib().orc_quant_blocks(_ptr(x), rows, cols, cols, blk, blk, _ptr(codes), _ptr(scales))
    return codes, scales


def linear_w8a8(xq, sx, wq, sw, bias_bits=None, blk: int = LINEAR_BLK):
    """W8A8 linear y = sum_kb s_x s_w S_kb + b in fp64.  xq [M, K] int8 with sx [ceil(M/blk), K/blk]; wq [N, K]
    with sw [ceil(N/blk), K/blk]; bias: bf16 patterns [N] or None.  Returns (y [M, N], mag [M, N])."""
    xq, wq = _dense(xq, np.int8), _dense(wq, np.int8)
    sx, sw = _dense(sx, np.float32), _dense(sw, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and K % blk == 0
    assert sx.shape == (_nblk(M, blk), K // blk) and sw.shape == (_nblk(N, blk), K // blk)
    b = None if bias_bits is None else _dense(np.asarray(bias_bits), np.uint16)
    assert b is None or b.shape == (N,)
    y = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    lib().orc_linear_w8a8(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(b), M, N, K, blk, _ptr(y), _ptr(mag))
    return y, mag


def linear_w8a16(x_bits, wq, sw, bias_bits=None, blk: int = LINEAR_BLK):
    """W8A16 linear y = sum_kb s_w (x . Wq)_kb + b in fp64.  x: bf16 patterns [M, K]; wq, sw, bias as for
    linear_w8a8.  Returns (y [M, N], mag [M, N])."""
    x, wq, sw = _dense(np.asarray(x_bits), np.uint16), _dense(wq, np.int8), _dense(sw, np.float32)
    M, K = x.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and K % blk == 0 and sw.shape == (_nblk(N, blk), K // blk)
    b = None if bias_bits is None else _dense(np.asarray(bias_bits), np.uint16)
    assert b is None or b.shape == (N,)
    y = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    lib().orc_linear_w8a16(_ptr(x), _ptr(wq), _ptr(sw), _ptr(b), M, N, K, blk, _ptr(y), _ptr(mag))
    return y, mag
