"""Python binding of libdca.so: argument marshalling only.

Each function has the name of the C entry point it calls (without the ``dca_`` prefix) and takes
torch tensors that already live on the GPU.  PyTorch provides the device memory and the current
stream; every step of the computation runs in the library's HIP kernels.  If the library is
missing this module raises: there is no other implementation to fall back to.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdca.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(5)
F32, BF16 = 0, 1
INTRA, SUCC, INTER = 0, 1, 2
REMAP_BASELINE, REMAP_PAGE_C, REMAP_PAGE_2C = 0, 1, 2   # dca_remap_mode
KV_BF16, KV_Q8_0, KV_Q4_0 = 0, 1, 2                    # dca_kv_format
MAX_MERGE_PARTS = 8


class DcaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"dca status {status}: {msg}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("n_rot", ctypes.c_int32),
                ("n_head_q", ctypes.c_int32), ("n_head_kv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("remap_mode", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("scale", ctypes.c_float),
                ("freq_factors", ctypes.c_void_p), ("rope_attn_factor", ctypes.c_float)]


class _Region(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int), ("keys", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("n", ctypes.c_int32)]


_lib = None


def lib():
    """Load libdca.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with dual_chunk_attention_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(_Config)
        L.dca_remap_positions.argtypes = [cfgp, i32, i32, vp, i32, vp, vp, vp, vp]
        L.dca_rope_partial.argtypes = [cfgp, ctypes.c_int, vp, i64, i32, vp, vp, vp]
        L.dca_attn_regime.argtypes = [cfgp, ctypes.c_int, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp,
                                      vp, sz, vp]
        L.dca_attn_regime_workspace_size.argtypes = [cfgp, ctypes.c_int, i32, i32, i32]
        L.dca_attn_regime_workspace_size.restype = sz
        L.dca_lse_merge.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i64, i32,
                                    ctypes.c_int, vp, vp, vp]
        L.dca_attention.argtypes = [cfgp, ctypes.c_int, i32, i32, vp, vp, vp, i32, ctypes.c_int, vp,
                                    vp, vp, sz, vp]
        L.dca_attention_noalloc.argtypes = [cfgp, ctypes.c_int, i32, i32, vp, vp, vp, i32, ctypes.c_int, vp,
                                            vp, vp]
        L.dca_attention_workspace_size.argtypes = [cfgp, ctypes.c_int, i32, i32, i32]
        L.dca_attention_workspace_size.restype = sz
        L.dca_attention_q8.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, i32, ctypes.c_int, vp, vp, vp,
                                       sz, vp]
        L.dca_attention_q8_workspace_size.argtypes = [cfgp, i32, i32, i32]
        L.dca_attention_q8_workspace_size.restype = sz
        L.dca_attention_q4.argtypes = L.dca_attention_q8.argtypes
        L.dca_attention_q4_workspace_size.argtypes = [cfgp, i32, i32, i32]
        L.dca_attention_q4_workspace_size.restype = sz
        regp = ctypes.POINTER(_Region)
        L.dca_attention_window.argtypes = [cfgp, i32, i32, vp, vp, regp, regp, ctypes.c_int, vp, vp,
                                           vp, sz, vp]
        L.dca_attention_window_workspace_size.argtypes = [cfgp, i32, i32, i32, i32]
        L.dca_attention_window_workspace_size.restype = sz
        L.dca_set_stage_events.argtypes = [vp, i32]
        L.dca_set_stage_events.restype = ctypes.c_int
        L.dca_last_error.restype = ctypes.c_char_p
        L.dca_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
        L.dca_probe_hbm_read.argtypes = [vp, i64, i32, vp, vp]
        for f in ("dca_remap_positions", "dca_rope_partial", "dca_attn_regime", "dca_lse_merge",
                  "dca_attention", "dca_attention_noalloc", "dca_attention_q8", "dca_attention_q4", "dca_attention_window",
                  "dca_probe_mfma_bf16", "dca_probe_hbm_read"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


@dataclass
class Config:
    """Mirror of dca_config (include/dca.h).  freq_factors: fp32 CUDA tensor [n_rot/2] or None."""
    head_dim: int = 512
    n_rot: int = 128
    n_head_q: int = 16
    n_head_kv: int = 2
    chunk: int = 8192
    rope_theta: float = 1.0e6
    scale: Optional[float] = None
    freq_factors: Optional[torch.Tensor] = None
    remap_mode: int = 0
    rope_attn_factor: float = 1.0

    def c(self):
        scale = self.scale if self.scale is not None else (self.head_dim ** -0.5 if self.head_dim > 0 else 1.0)
        ff = 0
        if self.freq_factors is not None:
            assert self.freq_factors.dtype == torch.float32 and self.freq_factors.is_contiguous()
            ff = self.freq_factors.data_ptr()
        return _Config(self.head_dim, self.n_rot, self.n_head_q, self.n_head_kv, self.chunk,
                       self.remap_mode, self.rope_theta, scale, ff, self.rope_attn_factor)


def _check(status):
    if status != OK:
        raise DcaError(status, lib().dca_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def remap_positions(cfg: Config, q_pos: torch.Tensor, n_kv: int, want_pos_k: bool = True):
    """dca_remap_positions: q_pos int32 [B,T] -> (pos_q [3,B,T], pos_k [n_kv], bounds [3,B,T,2])."""
    assert q_pos.dtype == torch.int32 and q_pos.is_contiguous() and q_pos.dim() == 2
    B, T = q_pos.shape
    dev = q_pos.device
    pos_q = torch.empty((3, B, T), dtype=torch.int32, device=dev)
    pos_k = torch.empty((n_kv,), dtype=torch.int32, device=dev) if want_pos_k else None
    bounds = torch.empty((3, B, T, 2), dtype=torch.int32, device=dev)
    c = cfg.c()
    _check(lib().dca_remap_positions(ctypes.byref(c), B, T, _ptr(q_pos), n_kv, _ptr(pos_q),
                                     _ptr(pos_k), _ptr(bounds), _stream()))
    return pos_q, pos_k, bounds


def rope_partial(cfg: Config, x: torch.Tensor, pos: torch.Tensor, out: Optional[torch.Tensor] = None):
    """dca_rope_partial: x [rows, H, D] (bf16 or fp32), pos int32 [rows] -> y (may be x)."""
    assert x.is_contiguous() and x.dim() == 3 and x.shape[2] == cfg.head_dim
    assert pos.dtype == torch.int32 and pos.is_contiguous() and pos.numel() == x.shape[0]
    y = torch.empty_like(x) if out is None else out
    c = cfg.c()
    _check(lib().dca_rope_partial(ctypes.byref(c), _dtype_code(x.dtype), _ptr(x), x.shape[0],
                                  x.shape[1], _ptr(pos), _ptr(y), _stream()))
    return y


def attn_regime(cfg: Config, regime: int, q_r: torch.Tensor, bounds: torch.Tensor,
                k_rot: torch.Tensor, k_raw: torch.Tensor):
    """dca_attn_regime: q_r [B,T,Hq,D], bounds [3,B,T,2], k_rot [B,N,Hkv,n_rot] (the rotary dims
    of the rotated keys), k_raw [B,N,Hkv,D] -> (o_r fp32 [B,T,Hq,D], lse_r fp32 [B,T,Hq])."""
    B, T, Hq, D = q_r.shape
    N = k_raw.shape[1]
    assert k_rot.shape == (B, N, k_raw.shape[2], cfg.n_rot), (tuple(k_rot.shape), cfg.n_rot)
    for t in (q_r, bounds, k_rot, k_raw):
        assert t.is_contiguous()
    dt = _dtype_code(q_r.dtype)
    c = cfg.c()
    ws_bytes = lib().dca_attn_regime_workspace_size(ctypes.byref(c), dt, B, T, N)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=q_r.device)
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q_r.device)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q_r.device)
    _check(lib().dca_attn_regime(ctypes.byref(c), dt, regime, B, T, _ptr(q_r), _ptr(bounds),
                                 _ptr(k_rot), _ptr(k_raw), N, _ptr(o), _ptr(lse), _ptr(ws),
                                 ws_bytes, _stream()))
    return o, lse


def lse_merge(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor],
              out_dtype: torch.dtype = torch.float32):
    """dca_lse_merge: parts o_p fp32 [..., D], lse_p fp32 [...] -> (o [..., D], lse [...])."""
    n = len(o_parts)
    D = o_parts[0].shape[-1]
    rows = lse_parts[0].numel()
    for o, l in zip(o_parts, lse_parts):
        assert o.dtype == torch.float32 and l.dtype == torch.float32
        assert o.is_contiguous() and l.is_contiguous() and o.numel() == rows * D
    optr = (ctypes.c_void_p * n)(*[o.data_ptr() for o in o_parts])
    lptr = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lse_parts])
    out = torch.empty(o_parts[0].shape, dtype=out_dtype, device=o_parts[0].device)
    lse = torch.empty(lse_parts[0].shape, dtype=torch.float32, device=o_parts[0].device)
    _check(lib().dca_lse_merge(n, optr, lptr, rows, D, _dtype_code(out_dtype), _ptr(out), _ptr(lse),
                               _stream()))
    return out, lse


def attention_workspace_size(cfg: Config, dtype: torch.dtype, B: int, T: int, n_kv: int) -> int:
    c = cfg.c()
    return int(lib().dca_attention_workspace_size(ctypes.byref(c), _dtype_code(dtype), B, T, n_kv))


def attention(cfg: Config, q: torch.Tensor, q_pos: torch.Tensor, k: torch.Tensor,
              o_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """dca_attention: q [B,T,Hq,D], q_pos int32 [B,T], k [B,N,Hkv,D] (K = V)
    -> (o [B,T,Hq,D] of o_dtype (default: q's dtype), lse fp32 [B,T,Hq])."""
    B, T, Hq, D = q.shape
    N = k.shape[1]
    assert q.is_contiguous() and k.is_contiguous() and q_pos.is_contiguous()
    assert q_pos.dtype == torch.int32 and q.dtype == k.dtype
    dt = _dtype_code(q.dtype)
    od = o_dtype or q.dtype
    c = cfg.c()
    ws_bytes = lib().dca_attention_workspace_size(ctypes.byref(c), dt, B, T, N)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=od, device=q.device)
    if lse is None:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    _check(lib().dca_attention(ctypes.byref(c), dt, B, T, _ptr(q), _ptr(q_pos), _ptr(k), N,
                               _dtype_code(od), _ptr(out), _ptr(lse), _ptr(workspace),
                               workspace.numel(), _stream()))
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20   # DCA_NOALLOC_SCRATCH_BYTES of include/dca.h


def attention_noalloc(cfg: Config, q: torch.Tensor, q_pos: torch.Tensor, k: torch.Tensor,
                      out: torch.Tensor, lse: torch.Tensor):
    """dca_attention_noalloc: as attention(), with the library's static scratch as workspace; the
    caller passes the outputs (o [B,T,Hq,D] of the output dtype, lse fp32 [B,T,Hq])."""
    B, T, Hq, D = q.shape
    N = k.shape[1]
    for t in (q, k, q_pos, out, lse):
        assert t.is_contiguous()
    assert q_pos.dtype == torch.int32 and q.dtype == k.dtype and lse.dtype == torch.float32
    c = cfg.c()
    _check(lib().dca_attention_noalloc(ctypes.byref(c), _dtype_code(q.dtype), B, T, _ptr(q), _ptr(q_pos),
                                       _ptr(k), N, _dtype_code(out.dtype), _ptr(out), _ptr(lse), _stream()))
    return out, lse


def attention_q8_workspace_size(cfg: Config, B: int, T: int, n_kv: int) -> int:
    c = cfg.c()
    return int(lib().dca_attention_q8_workspace_size(ctypes.byref(c), B, T, n_kv))


def attention_q4_workspace_size(cfg: Config, B: int, T: int, n_kv: int) -> int:
    c = cfg.c()
    return int(lib().dca_attention_q4_workspace_size(ctypes.byref(c), B, T, n_kv))


def _attention_quant(fn, ws_fn, per_byte, code_dtypes, cfg, q, q_pos, k_codes, k_scales, o_dtype,
                     workspace, out, lse):
    B, T, Hq, D = q.shape
    N = k_codes.shape[1]
    assert q.dtype == torch.bfloat16 and q_pos.dtype == torch.int32
    assert k_codes.dtype in code_dtypes and k_scales.dtype in (torch.float16, torch.int16)
    assert k_codes.shape[3] * per_byte == D
    assert k_scales.shape == (*k_codes.shape[:3], D // 32)
    assert q.is_contiguous() and q_pos.is_contiguous()
    assert k_codes.is_contiguous() and k_scales.is_contiguous()
    od = o_dtype or torch.bfloat16
    c = cfg.c()
    ws_bytes = ws_fn(ctypes.byref(c), B, T, N)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=od, device=q.device)
    if lse is None:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    _check(fn(ctypes.byref(c), B, T, _ptr(q), _ptr(q_pos), _ptr(k_codes), _ptr(k_scales), N,
              _dtype_code(od), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse


def attention_q8(cfg: Config, q: torch.Tensor, q_pos: torch.Tensor, k_codes: torch.Tensor,
                 k_scales: torch.Tensor, o_dtype: Optional[torch.dtype] = None,
                 workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None):
    """dca_attention_q8: q bf16 [B,T,Hq,D], q_pos int32 [B,T], q8_0 key cache (K = V) as int8
    codes [B,N,Hkv,D] and fp16 scales [B,N,Hkv,D/32] (the scales' raw bits may also come as int16)
    -> (o [B,T,Hq,D] of o_dtype (default bf16), lse fp32 [B,T,Hq])."""
    L = lib()
    return _attention_quant(L.dca_attention_q8, L.dca_attention_q8_workspace_size, 1, (torch.int8,),
                            cfg, q, q_pos, k_codes, k_scales, o_dtype, workspace, out, lse)


def attention_q4(cfg: Config, q: torch.Tensor, q_pos: torch.Tensor, k_codes: torch.Tensor,
                 k_scales: torch.Tensor, o_dtype: Optional[torch.dtype] = None,
                 workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None):
    """dca_attention_q4: as attention_q8 over a q4_0 key cache: codes uint8 [B,N,Hkv,D/2] (dim 2j
    in the low nibble of byte j) and fp16 scales [B,N,Hkv,D/32]."""
    L = lib()
    return _attention_quant(L.dca_attention_q4, L.dca_attention_q4_workspace_size, 2, (torch.uint8,),
                            cfg, q, q_pos, k_codes, k_scales, o_dtype, workspace, out, lse)


@dataclass
class Region:
    """One region of a key cache for attention_window: format KV_BF16 (keys bf16 [B,n,Hkv,D]),
    KV_Q8_0 (int8 codes [B,n,Hkv,D] + fp16/int16 scales [B,n,Hkv,D/32]) or KV_Q4_0 (uint8 codes
    [B,n,Hkv,D/2] + scales).  The tensors may live on the GPU or in pinned host memory
    (torch's pin_memory=True)."""
    format: int
    keys: Optional[torch.Tensor]
    scales: Optional[torch.Tensor] = None

    def n(self) -> int:
        return 0 if self.keys is None else int(self.keys.shape[1])

    def c(self):
        if self.keys is not None:
            assert self.keys.is_contiguous() and (self.scales is None or self.scales.is_contiguous())
        return _Region(self.format, None if self.keys is None else self.keys.data_ptr(),
                       None if self.scales is None else self.scales.data_ptr(), self.n())


def attention_window_workspace_size(cfg: Config, B: int, T: int, n_win: int, n_tail: int) -> int:
    c = cfg.c()
    return int(lib().dca_attention_window_workspace_size(ctypes.byref(c), B, T, n_win, n_tail))


def attention_window(cfg: Config, q: torch.Tensor, q_pos: torch.Tensor, window: Region, tail: Region,
                     o_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """dca_attention_window: q bf16 [B,T,Hq,D] on the GPU, q_pos int32 [B,T]; cells
    [0, window.n) of the cache from `window`, [window.n, window.n + tail.n) from `tail` ->
    (o [B,T,Hq,D] of o_dtype (default bf16), lse fp32 [B,T,Hq])."""
    B, T, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q_pos.dtype == torch.int32
    assert q.is_contiguous() and q_pos.is_contiguous()
    od = o_dtype or torch.bfloat16
    c = cfg.c()
    ws_bytes = lib().dca_attention_window_workspace_size(ctypes.byref(c), B, T, window.n(), tail.n())
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=od, device=q.device)
    if lse is None:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    rw, rt = window.c(), tail.c()
    _check(lib().dca_attention_window(ctypes.byref(c), B, T, _ptr(q), _ptr(q_pos), ctypes.byref(rw),
                                      ctypes.byref(rt), _dtype_code(od), _ptr(out), _ptr(lse),
                                      _ptr(workspace), workspace.numel(), _stream()))
    return out, lse


N_STAGE_EVENTS = 6


def set_stage_events(events_array) -> None:
    """dca_set_stage_events: `events_array` is a ctypes array of >= 6 hipEvent_t handles created by
    the caller (None turns the hook off).  Later dca_attention calls on this thread record them
    around their stages."""
    if events_array is None:
        _check(lib().dca_set_stage_events(None, 0))
    else:
        _check(lib().dca_set_stage_events(ctypes.cast(events_array, ctypes.c_void_p), len(events_array)))


def probe_mfma_bf16(n_workgroups: int, iters: int, sink: torch.Tensor) -> None:
    """dca_probe_mfma_bf16 (include/dca_calibrate.h): matrix-core loop on the current stream;
    sink fp32 [n_workgroups * 256]."""
    assert sink.dtype == torch.float32 and sink.numel() >= n_workgroups * 256
    _check(lib().dca_probe_mfma_bf16(n_workgroups, iters, _ptr(sink), _stream()))


def probe_hbm_read(src: torch.Tensor, n_workgroups: int, sink: torch.Tensor) -> None:
    """dca_probe_hbm_read: streaming read of src's bytes on the current stream."""
    assert src.is_contiguous() and sink.dtype == torch.float32 and sink.numel() >= n_workgroups * 256
    _check(lib().dca_probe_hbm_read(_ptr(src), src.numel() * src.element_size(), n_workgroups,
                                    _ptr(sink), _stream()))
