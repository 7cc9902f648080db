"""CPU oracle for Dual Chunk Attention: thin ctypes wrapper over the fp64 C code in dca_oracle.c.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's CPU-baseline leg may
import this package; the GPU library neither imports nor links it, and it imports nothing from
the GPU library.  Every function below states the passage of the pages it follows (see the header
of dca_oracle.c for the remap and RoPE readings it fixes).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

INTRA, SUCC, INTER = 0, 1, 2
# remap modes: the reading fixed in dca_oracle.c, then the page-literal tables (inter query at c,
# inter query at 2c; succ = the whole previous chunk in both)
REMAP_BASELINE, REMAP_PAGE_C, REMAP_PAGE_2C = 0, 1, 2


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        i64, i32p, f64p = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)
        lib.dca_oracle_regime.restype = ctypes.c_int
        lib.dca_oracle_regime.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        lib.dca_oracle_query_pos.restype = i64
        lib.dca_oracle_query_pos.argtypes = [i64, i64, ctypes.c_int, ctypes.c_int]
        lib.dca_oracle_key_pos.restype = i64
        lib.dca_oracle_key_pos.argtypes = [i64, i64]
        lib.dca_oracle_remap.restype = i64
        lib.dca_oracle_remap.argtypes = [i64, ctypes.c_int, i64, i32p, i64, i32p, i32p, i32p, ctypes.c_int]
        lib.dca_oracle_rope.restype = None
        lib.dca_oracle_rope.argtypes = [i64, i64, ctypes.c_double, f64p, f64p,
                                        ctypes.POINTER(ctypes.c_int64), i64, i64, f64p, ctypes.c_double]
        lib.dca_oracle_merge.restype = None
        lib.dca_oracle_merge.argtypes = [i64, f64p, f64p, i64, i64, f64p, f64p]
        lib.dca_oracle_attention.restype = ctypes.c_int
        lib.dca_oracle_attention.argtypes = [
            i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_double, ctypes.c_double, f64p, ctypes.c_int,
            ctypes.c_int, i64, i64, ctypes.c_void_p, i32p, ctypes.c_void_p, i64, i64,
            ctypes.POINTER(ctypes.c_int64), f64p, f64p, f64p, f64p, ctypes.c_int, ctypes.c_double]
        lib.dca_oracle_attention_q8.restype = ctypes.c_int
        lib.dca_oracle_attention_q8.argtypes = [
            i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_double, ctypes.c_double, f64p, ctypes.c_int,
            i64, i64, ctypes.c_void_p, i32p, ctypes.c_void_p, ctypes.c_void_p, i64, i64,
            ctypes.POINTER(ctypes.c_int64), f64p, f64p, f64p, f64p, ctypes.c_int, ctypes.c_double]
        lib.dca_oracle_half.restype = ctypes.c_double
        lib.dca_oracle_half.argtypes = [ctypes.c_uint16]
        lib.dca_oracle_dequant_q8.restype = None
        lib.dca_oracle_dequant_q8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, f64p]
        lib.dca_oracle_attention_q4.restype = ctypes.c_int
        lib.dca_oracle_attention_q4.argtypes = lib.dca_oracle_attention_q8.argtypes
        lib.dca_oracle_dequant_q4.restype = None
        lib.dca_oracle_dequant_q4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, f64p]
        _LIB = lib
    return _LIB


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def regime(i, j, c, n_kv, mode=REMAP_BASELINE):
    """Regime of key j for a query at i (DCA feature page, "Section C design" table, read as in
    the header of dca_oracle.c, or literally for the page modes); -1 when the key is not attended."""
    return _lib().dca_oracle_regime(int(i), int(j), int(c), int(n_kv), int(mode))


def query_pos(i, c, r, mode=REMAP_BASELINE):
    """Remapped query position of regime r (intra i mod c, succ (i mod c)+c, inter c-1; the page
    modes put inter at c or 2c)."""
    return _lib().dca_oracle_query_pos(int(i), int(c), int(r), int(mode))


def key_pos(j, c):
    """Key position j mod c (rope-K-once, "Section C design")."""
    return _lib().dca_oracle_key_pos(int(j), int(c))


def remap(c, qpos, n_kv, n_threads=0, mode=REMAP_BASELINE):
    """Positions and per-regime key intervals by enumeration of the explicit predicate.

    Returns (pos_q int32 [3, rows], pos_k int32 [n_kv], bounds int32 [3, rows, 2], status);
    status 0 means every regime key set was one contiguous interval."""
    qpos = np.ascontiguousarray(np.asarray(qpos, dtype=np.int32).reshape(-1))
    rows = qpos.size
    pos_q = np.zeros((3, rows), np.int32)
    pos_k = np.zeros((max(n_kv, 0),), np.int32)
    bounds = np.zeros((3, rows, 2), np.int32)
    st = _lib().dca_oracle_remap(int(c), int(mode), rows, _ptr(qpos, ctypes.c_int32), int(n_kv),
                                 _ptr(pos_q, ctypes.c_int32), _ptr(pos_k, ctypes.c_int32),
                                 _ptr(bounds, ctypes.c_int32), int(n_threads))
    return pos_q, pos_k, bounds, int(st)


def rope(x, pos, n_rot, theta, freq_factors=None, attn_factor=1.0):
    """Partial RoPE of x [rows, H, D] (fp64) at integer positions pos [rows] ("DCA algorithm":
    only the rotary dims move; proportional rope with freq_factors, "Why llamafile is
    sufficient"); attn_factor multiplies the rotated dims (YaRN magnitude, 1 = none)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, H, D = x.shape
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64).reshape(rows))
    y = np.empty_like(x)
    ff = None if freq_factors is None else np.ascontiguousarray(freq_factors, dtype=np.float64)
    _lib().dca_oracle_rope(int(n_rot), D, float(theta), None if ff is None else _ptr(ff, ctypes.c_double),
                           _ptr(x, ctypes.c_double), _ptr(pos, ctypes.c_int64), rows, H,
                           _ptr(y, ctypes.c_double), float(attn_factor))
    return y


def merge(o_parts, lse_parts):
    """N-way LSE merge (Implementation progress + Section-D simplification).
    o_parts [P, rows, D], lse_parts [P, rows] -> (o [rows, D], lse [rows])."""
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    P, rows, D = o_parts.shape
    o = np.empty((rows, D), np.float64)
    lse = np.empty((rows,), np.float64)
    _lib().dca_oracle_merge(P, _ptr(o_parts, ctypes.c_double), _ptr(lse_parts, ctypes.c_double),
                            rows, D, _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return o, lse


def attention(q, qpos, k, *, chunk, n_rot, theta, scale, freq_factors=None, rows=None,
              per_regime=True, n_threads=0, round_rotated_bf16=False, remap_mode=REMAP_BASELINE,
              attn_factor=1.0):
    """DCA attention of selected query rows in fp64.

    q [B, T, Hq, D] and k [B, N, Hkv, D] are float32 arrays or uint16 bf16 bit patterns (same
    kind for both); qpos int32 [B, T]; rows = flat row indices b*T+t (default: all).
    round_rotated_bf16: round the rotated dims of queries and keys to bf16 before the scores
    (the contract of a caller passing bf16 rotated operands to the per-regime entry point).
    remap_mode: REMAP_BASELINE (the reading of dca_oracle.c) or a page-literal mode.
    Returns dict(o [n, Hq, D], lse [n, Hq], o_reg [3, n, Hq, D], lse_reg [3, n, Hq], rows)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    if q.dtype == np.uint16 and k.dtype == np.uint16:
        in_bf16 = 1
    elif q.dtype == np.float32 and k.dtype == np.float32:
        in_bf16 = 0
    else:
        raise TypeError("q and k must both be float32 or both uint16 (bf16 bits)")
    B, T, Hq, D = q.shape
    Bk, N, Hkv, Dk = k.shape
    assert Bk == B and Dk == D
    qpos = np.ascontiguousarray(np.asarray(qpos, dtype=np.int32).reshape(B, T))
    sel = np.arange(B * T, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = sel.size
    o = np.zeros((n, Hq, D), np.float64)
    lse = np.zeros((n, Hq), np.float64)
    o_reg = np.zeros((3, n, Hq, D), np.float64) if per_regime else None
    lse_reg = np.zeros((3, n, Hq), np.float64) if per_regime else None
    ff = None if freq_factors is None else np.ascontiguousarray(freq_factors, dtype=np.float64)
    st = _lib().dca_oracle_attention(
        D, int(n_rot), Hq, Hkv, int(chunk), int(remap_mode), float(theta), float(scale),
        None if ff is None else _ptr(ff, ctypes.c_double), in_bf16, 1 if round_rotated_bf16 else 0, B, T,
        q.ctypes.data_as(ctypes.c_void_p), _ptr(qpos, ctypes.c_int32),
        k.ctypes.data_as(ctypes.c_void_p), N, n, _ptr(sel, ctypes.c_int64),
        _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
        None if o_reg is None else _ptr(o_reg, ctypes.c_double),
        None if lse_reg is None else _ptr(lse_reg, ctypes.c_double), int(n_threads), float(attn_factor))
    if st != 0:
        raise RuntimeError(f"oracle attention failed with status {st}")
    return dict(o=o, lse=lse, o_reg=o_reg, lse_reg=lse_reg, rows=sel)


def half(bits):
    """Value of IEEE binary16 bit patterns (the q8_0 block scale), by the format's definition."""
    return _lib().dca_oracle_half(int(bits) & 0xFFFF)


def dequant_q8(codes, scales):
    """Values d * q of a q8_0 cache (reading in the header of dca_oracle.c): codes int8 [..., D],
    scales uint16 fp16 bits [..., D/32] -> float64 [..., D]."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    assert codes.shape[:-1] == scales.shape[:-1] and codes.shape[-1] == 32 * scales.shape[-1]
    out = np.empty(codes.shape, np.float64)
    _lib().dca_oracle_dequant_q8(codes.ctypes.data_as(ctypes.c_void_p), scales.ctypes.data_as(ctypes.c_void_p),
                                 codes.size, _ptr(out, ctypes.c_double))
    return out


def dequant_q4(codes, scales):
    """Values d * (n - 8) of a q4_0 cache (reading in the header of dca_oracle.c): codes uint8
    [..., D/2] (dim 2j in the low nibble of byte j), scales uint16 fp16 bits [..., D/32] ->
    float64 [..., D]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    assert codes.shape[:-1] == scales.shape[:-1] and 2 * codes.shape[-1] == 32 * scales.shape[-1]
    out = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), np.float64)
    _lib().dca_oracle_dequant_q4(codes.ctypes.data_as(ctypes.c_void_p), scales.ctypes.data_as(ctypes.c_void_p),
                                 out.size, _ptr(out, ctypes.c_double))
    return out


def _attention_quant(fn, elems_per_byte, code_dtype, q, qpos, codes, scales, *, chunk, n_rot, theta,
                     scale, freq_factors, rows, per_regime, n_threads, remap_mode, attn_factor):
    q = np.ascontiguousarray(q)
    codes = np.ascontiguousarray(codes, dtype=code_dtype)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if q.dtype == np.uint16:
        q_bf16 = 1
    elif q.dtype == np.float32:
        q_bf16 = 0
    else:
        raise TypeError("q must be float32 or uint16 (bf16 bits)")
    B, T, Hq, D = q.shape
    Bk, N, Hkv, Dk = codes.shape
    assert Bk == B and Dk * elems_per_byte == D and scales.shape == (B, N, Hkv, D // 32)
    qpos = np.ascontiguousarray(np.asarray(qpos, dtype=np.int32).reshape(B, T))
    sel = np.arange(B * T, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = sel.size
    o = np.zeros((n, Hq, D), np.float64)
    lse = np.zeros((n, Hq), np.float64)
    o_reg = np.zeros((3, n, Hq, D), np.float64) if per_regime else None
    lse_reg = np.zeros((3, n, Hq), np.float64) if per_regime else None
    ff = None if freq_factors is None else np.ascontiguousarray(freq_factors, dtype=np.float64)
    st = fn(
        D, int(n_rot), Hq, Hkv, int(chunk), int(remap_mode), float(theta), float(scale),
        None if ff is None else _ptr(ff, ctypes.c_double), q_bf16, B, T,
        q.ctypes.data_as(ctypes.c_void_p), _ptr(qpos, ctypes.c_int32),
        codes.ctypes.data_as(ctypes.c_void_p), scales.ctypes.data_as(ctypes.c_void_p), N, n,
        _ptr(sel, ctypes.c_int64), _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
        None if o_reg is None else _ptr(o_reg, ctypes.c_double),
        None if lse_reg is None else _ptr(lse_reg, ctypes.c_double), int(n_threads), float(attn_factor))
    if st != 0:
        raise RuntimeError(f"oracle attention failed with status {st}")
    return dict(o=o, lse=lse, o_reg=o_reg, lse_reg=lse_reg, rows=sel)


def attention_q8(q, qpos, codes, scales, *, chunk, n_rot, theta, scale, freq_factors=None, rows=None,
                 per_regime=True, n_threads=0, remap_mode=REMAP_BASELINE, attn_factor=1.0):
    """DCA attention (as `attention`) over a q8_0 key cache: codes int8 [B, N, Hkv, D], scales
    uint16 fp16 bits [B, N, Hkv, D/32]; the keys (and values, K = V) are d * q.  q is float32 or
    uint16 bf16 bits [B, T, Hq, D]."""
    return _attention_quant(_lib().dca_oracle_attention_q8, 1, np.int8, q, qpos, codes, scales,
                            chunk=chunk, n_rot=n_rot, theta=theta, scale=scale, freq_factors=freq_factors,
                            rows=rows, per_regime=per_regime, n_threads=n_threads, remap_mode=remap_mode,
                            attn_factor=attn_factor)


def attention_q4(q, qpos, codes, scales, *, chunk, n_rot, theta, scale, freq_factors=None, rows=None,
                 per_regime=True, n_threads=0, remap_mode=REMAP_BASELINE, attn_factor=1.0):
    """DCA attention (as `attention`) over a q4_0 key cache: codes uint8 [B, N, Hkv, D/2] (two
    per byte), scales uint16 fp16 bits [B, N, Hkv, D/32]; the keys (and values) are d * (n - 8)."""
    return _attention_quant(_lib().dca_oracle_attention_q4, 2, np.uint8, q, qpos, codes, scales,
                            chunk=chunk, n_rot=n_rot, theta=theta, scale=scale, freq_factors=freq_factors,
                            rows=rows, per_regime=per_regime, n_threads=n_threads, remap_mode=remap_mode,
                            attn_factor=attn_factor)
