"""Seeded synthetic inputs for Dual Chunk Attention workloads.

This module holds no arithmetic of the method: it only draws inputs, rounds them to bf16 and, for
the quantized-cache workloads, stores the keys as q8_0 blocks.  Both the GPU path (tests,
benchmark) and the CPU oracle read the bytes it produces.

Recipe: numpy ``default_rng(seed)``; draw Q, then K, then freq_factors; Q and K are i.i.d.
standard normal float32 (unit RMS, as after q/k-norm), rounded to bf16 by round-to-nearest-even
for bf16 workloads; freq_factors are float32 uniform in [1, 8) (all 1.0 for the fp32 workload).
Keys are cache cells 0..N-1 at positions equal to their index; prefill queries are the positions
listed per workload; decode queries sit at N-1.

q8_0 workloads (dtype "q8_0"): Q as for bf16; K drawn as float32 and stored as q8_0 blocks of 32
consecutive dims of a (key, KV head) row: scale d = max|x| / 127 stored as fp16 (nearest-even),
codes q = x / d rounded half away from zero (from the unrounded d; 0 for an all-zero block).  The
cache is int8 codes [B,N,Hkv,D] plus fp16 scales [B,N,Hkv,D/32]; its values are fp16(d) * q.

q4_0 workloads (dtype "q4_0"): the same draws stored as q4_0 blocks of 32 dims: d = max|x| / 7 as
fp16, codes n = round-half-away(x / d) + 8 in [1, 15] (8 for an all-zero block), packed two per
byte in dim order (dim 2j in the low nibble of byte j): uint8 codes [B,N,Hkv,D/2] plus fp16 scales
[B,N,Hkv,D/32]; values fp16(d) * (n - 8).
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    q0: int            # first query position; query t of every sequence sits at q0 + t
    N: int             # KV cache length per sequence
    chunk: int
    Hq: int
    Hkv: int
    dtype: str         # "f32", "bf16", "q8_0" or "q4_0"
    seed: int
    D: int = 512
    n_rot: int = 128
    theta: float = 1.0e6
    ff_uniform: bool = True   # freq_factors ~ U[1,8); False -> all 1.0
    notes: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.D))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("prefill-256-c64-fp32", 1, 256, 0, 256, 64, 2, 1, "f32", 1, ff_uniform=False,
                 notes="tiny single global layer, fp32, all three regimes"),
        Workload("prefill-4k-c1024", 1, 4096, 0, 4096, 1024, 16, 2, "bf16", 2),
        Workload("prefill-32k-c8192", 1, 32768, 0, 32768, 8192, 16, 2, "bf16", 3),
        Workload("decode-b8-kv256k-c65536", 8, 1, 262143, 262144, 65536, 16, 2, "bf16", 4),
        Workload("prefill-4k-at-1m-c65536", 1, 4096, 1044480, 1048576, 65536, 16, 2, "bf16", 5),
        Workload("decode-b8-kv256k-c65536-q8", 8, 1, 262143, 262144, 65536, 16, 2, "q8_0", 4,
                 notes="the 256k decode over a q8_0 key cache"),
        Workload("decode-b8-kv256k-c65536-q4", 8, 1, 262143, 262144, 65536, 16, 2, "q4_0", 4,
                 notes="the 256k decode over a q4_0 key cache"),
    ]
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, as_bf16, chunk_elems=1 << 24):
    """Standard normal float32 of `shape`, drawn in chunks (same stream as one draw)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16 if as_bf16 else np.float32)
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        v = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = bf16_bits(v) if as_bf16 else v
    return out.reshape(shape)


def q8_0_blocks(x: np.ndarray):
    """Store float32 x [..., D] (D a multiple of 32) as q8_0 blocks: (codes int8 [..., D],
    scales uint16 fp16 bits [..., D/32]); see the module docstring."""
    x = np.asarray(x, dtype=np.float32)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    d = np.abs(blk).max(axis=-1) / np.float32(127.0)
    inv = np.where(d > 0, np.float32(1.0) / np.where(d > 0, d, np.float32(1.0)), np.float32(0.0))
    v = blk * inv[..., None]
    codes = np.trunc(v + np.copysign(np.float32(0.5), v)).astype(np.int8)
    scales = d.astype(np.float16).view(np.uint16)
    return codes.reshape(x.shape), scales


def q4_0_blocks(x: np.ndarray):
    """Store float32 x [..., D] (D a multiple of 32) as q4_0 blocks: (codes uint8 [..., D/2], two
    per byte, scales uint16 fp16 bits [..., D/32]); see the module docstring."""
    x = np.asarray(x, dtype=np.float32)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    d = np.abs(blk).max(axis=-1) / np.float32(7.0)
    inv = np.where(d > 0, np.float32(1.0) / np.where(d > 0, d, np.float32(1.0)), np.float32(0.0))
    v = blk * inv[..., None]
    n = np.clip(np.trunc(v + np.copysign(np.float32(0.5), v)) + 8, 0, 15).astype(np.uint8)
    n = n.reshape(x.shape)
    codes = (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)
    scales = d.astype(np.float16).view(np.uint16)
    return codes, scales


def _normal_quant(rng, shape, blocks, code_div, code_dtype, chunk_elems=1 << 22):
    """Standard normal float32 of `shape` (same stream as _normal), stored by `blocks` (codes of
    D / code_div bytes per row + fp16 scales).  The draws stay sequential; the blocks are formed on
    a few threads."""
    from concurrent.futures import ThreadPoolExecutor

    n = int(np.prod(shape))
    D = shape[-1]
    codes = np.empty(n // code_div, code_dtype)
    scales = np.empty(n // 32, np.uint16)
    step = chunk_elems - chunk_elems % D

    def work(s, x):
        c, sc = blocks(x.reshape(-1, D))
        codes[s // code_div:(s + x.size) // code_div] = c.reshape(-1)
        scales[s // 32:(s + x.size) // 32] = sc.reshape(-1)

    with ThreadPoolExecutor(max_workers=8) as ex:
        futs = [ex.submit(work, s, rng.standard_normal(min(n, s + step) - s, dtype=np.float32))
                for s in range(0, n, step)]
        for f in futs:
            f.result()
    return codes.reshape(shape[:-1] + (D // code_div,)), scales.reshape(shape[:-1] + (D // 32,))


def _normal_q8(rng, shape, chunk_elems=1 << 22):
    return _normal_quant(rng, shape, q8_0_blocks, 1, np.int8, chunk_elems)


def _normal_q4(rng, shape, chunk_elems=1 << 22):
    return _normal_quant(rng, shape, q4_0_blocks, 2, np.uint8, chunk_elems)


def make_inputs(w, *, B=None, T=None, q0=None, N=None, seed=None):
    """Inputs of workload `w` (a Workload or its name); size overrides give smaller cases of the
    same recipe.  Returns dict(q, k, q_pos, freq_factors, w): q [B,T,Hq,D], k [B,N,Hkv,D] as
    uint16 bf16 bits (bf16 workloads) or float32; q_pos int32 [B,T]; freq_factors float32
    [n_rot/2].  q8_0 workloads: k is None and k_codes int8 [B,N,Hkv,D], k_scales uint16 fp16
    bits [B,N,Hkv,D/32] hold the cache; q4_0 workloads: k_codes uint8 [B,N,Hkv,D/2]."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    T = w.T if T is None else T
    q0 = w.q0 if q0 is None else q0
    N = w.N if N is None else N
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    as_bf16 = w.dtype in ("bf16", "q8_0", "q4_0")
    q = _normal(rng, (B, T, w.Hq, w.D), as_bf16)
    k = k_codes = k_scales = None
    if w.dtype == "q8_0":
        k_codes, k_scales = _normal_q8(rng, (B, N, w.Hkv, w.D))
    elif w.dtype == "q4_0":
        k_codes, k_scales = _normal_q4(rng, (B, N, w.Hkv, w.D))
    else:
        k = _normal(rng, (B, N, w.Hkv, w.D), as_bf16)
    if w.ff_uniform:
        ff = rng.uniform(1.0, 8.0, w.n_rot // 2).astype(np.float32)
    else:
        ff = np.ones(w.n_rot // 2, np.float32)
    q_pos = (q0 + np.arange(T, dtype=np.int64)).astype(np.int32)
    q_pos = np.ascontiguousarray(np.broadcast_to(q_pos, (B, T)))
    out = dict(q=q, k=k, q_pos=q_pos, freq_factors=ff, w=w)
    if k_codes is not None:
        out.update(k_codes=k_codes, k_scales=k_scales)
    return out
