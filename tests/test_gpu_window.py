"""GPU parity of the window + tail decode (dca_attention_window): a key cache split into a window
of cells [0, n_win) and a tail [n_win, n_kv), each region in its own format and either on the GPU
or in pinned host memory (read by the kernels over the host link).  The oracle is plain attention
over the whole cache: the split changes only where the bytes live.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from dual_chunk_attention_amd import dca, synth
from gpu_util import assert_lse_close, assert_o_close, cfg_for, dev, rows_of, to_dev

pytestmark = pytest.mark.gpu

FMT = {"bf16": dca.KV_BF16, "q8": dca.KV_Q8_0, "q4": dca.KV_Q4_0}


def _region(fmt, kf32, where):
    """Store float32 keys [B, n, Hkv, D] in format `fmt` on the GPU or in pinned host memory.
    Returns (dca.Region, the exact float32 values the region holds)."""
    if kf32.shape[1] == 0:
        return dca.Region(FMT[fmt], None, None), kf32
    if fmt == "bf16":
        bits = synth.bf16_bits(kf32)
        keys = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        scales, exact = None, synth.bf16_to_f32(bits)
    else:
        codes, sc = (synth.q8_0_blocks if fmt == "q8" else synth.q4_0_blocks)(kf32)
        keys = torch.from_numpy(codes)
        scales = torch.from_numpy(sc.view(np.int16))
        exact = (oracle.dequant_q8 if fmt == "q8" else oracle.dequant_q4)(codes, sc).astype(np.float32)
    move = (lambda t: t.to(dev())) if where == "device" else (lambda t: t.pin_memory())
    return dca.Region(FMT[fmt], move(keys), None if scales is None else move(scales)), exact


def _check(w, q_bits, q_pos, freq_factors, k_exact, out, rows=None, chunk=None, mode=0):
    o, lse = out
    torch.cuda.synchronize()
    ff = freq_factors.astype(np.float64)
    res = oracle.attention(synth.bf16_to_f32(q_bits), q_pos, k_exact, chunk=w.chunk if chunk is None else chunk,
                           n_rot=w.n_rot, theta=w.theta, scale=w.scale, freq_factors=ff, rows=rows,
                           per_regime=False, remap_mode=mode)
    B, T = q_bits.shape[:2]
    sel = res["rows"]
    got_o = o.float().cpu().numpy().reshape(B * T, w.Hq, w.D)[sel]
    got_l = lse.cpu().numpy().reshape(B * T, w.Hq)[sel]
    assert_o_close(got_o, res["o"])
    assert_lse_close(got_l, res["lse"])


CASES = [
    # (label, B, T, N, q0, n_win, chunk, window fmt, tail fmt, tail where, remap mode)
    ("bf16-bf16-host", 2, 1, 50000, 49999, 20000, 4096, "bf16", "bf16", "host", 0),
    ("q8-q4-host", 2, 1, 50000, 49999, 20000, 4096, "q8", "q4", "host", 0),
    ("q4-bf16-device", 2, 1, 30000, 29999, 12345, 4096, "q4", "bf16", "device", 0),
    ("all-tail-host", 1, 2, 9000, 8998, 0, 4096, "bf16", "q8", "host", 0),
    ("all-window", 1, 2, 9000, 8998, 9000, 4096, "q8", "bf16", "host", 0),
    ("t3-c3000-page2c", 1, 3, 9000, 8997, 4100, 3000, "q8", "bf16", "host", dca.REMAP_PAGE_2C),
    ("t8-succ-crosses", 1, 8, 9000, 8992, 7000, 2048, "bf16", "q4", "host", dca.REMAP_PAGE_C),
]


@pytest.mark.parametrize("label,B,T,N,q0,n_win,chunk,fw,ft,where,mode", CASES, ids=[c[0] for c in CASES])
def test_window_tail_decode(label, B, T, N, q0, n_win, chunk, fw, ft, where, mode):
    w = synth.Workload("win-" + label, B, T, q0, N, chunk, 16, 2, "bf16", 61)
    inp = synth.make_inputs(w, N=1)                        # q, q_pos and freq_factors
    kf = np.random.default_rng(62).standard_normal((B, N, 2, 512), dtype=np.float32)
    rw, ew = _region(fw, np.ascontiguousarray(kf[:, :n_win]), "device")
    rt, et = _region(ft, np.ascontiguousarray(kf[:, n_win:]), where)
    cfg = cfg_for(w, to_dev(inp["freq_factors"]), remap_mode=mode)
    out = dca.attention_window(cfg, to_dev(inp["q"]), to_dev(inp["q_pos"]), rw, rt, o_dtype=torch.float32)
    _check(w, inp["q"], inp["q_pos"], inp["freq_factors"], np.concatenate([ew, et], axis=1), out, mode=mode)


def test_window_tail_full_workload():
    """The 256k batch-8 decode with cells [0, 65536) on the GPU and [65536, 262144) in pinned host
    memory (bf16, 3.2 GB read over the host link), bf16 output; every head of rows 0, 5, 7."""
    w = synth.WORKLOADS["decode-b8-kv256k-c65536"]
    inp = synth.make_inputs(w)
    n_win = 65536
    k = torch.from_numpy(inp["k"].view(np.int16)).view(torch.bfloat16)
    rw = dca.Region(dca.KV_BF16, k[:, :n_win].contiguous().to(dev()))
    rt = dca.Region(dca.KV_BF16, k[:, n_win:].contiguous().pin_memory())
    cfg = cfg_for(w, to_dev(inp["freq_factors"]))
    o, lse = dca.attention_window(cfg, to_dev(inp["q"]), to_dev(inp["q_pos"]), rw, rt)
    torch.cuda.synchronize()
    rows = rows_of(w.B, w.T, [(0, 0), (5, 0), (7, 0)])
    res = oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=w.chunk, n_rot=w.n_rot, theta=w.theta,
                           scale=w.scale, freq_factors=inp["freq_factors"].astype(np.float64), rows=rows,
                           per_regime=False)
    assert_o_close(o.float().cpu().numpy().reshape(-1, w.Hq, w.D)[rows], res["o"])
    assert_lse_close(lse.cpu().numpy().reshape(-1, w.Hq)[rows], res["lse"])


def test_window_equals_whole_cache_decode():
    """The same bf16 cache as one device region and as window + host tail: both within the bar of
    each other (span boundaries differ, so not bit for bit)."""
    w = synth.WORKLOADS["decode-b8-kv256k-c65536"]
    inp = synth.make_inputs(w, B=2, N=40000, q0=39999)
    cfg = cfg_for(w, to_dev(inp["freq_factors"]))
    q, qp = to_dev(inp["q"]), to_dev(inp["q_pos"])
    k = torch.from_numpy(inp["k"].view(np.int16)).view(torch.bfloat16)
    o1, l1 = dca.attention(cfg, q, qp, k.to(dev()), o_dtype=torch.float32)
    o2, l2 = dca.attention_window(cfg, q, qp, dca.Region(dca.KV_BF16, k[:, :17000].contiguous().to(dev())),
                                  dca.Region(dca.KV_BF16, k[:, 17000:].contiguous().pin_memory()),
                                  o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_o_close(o2.cpu().numpy(), o1.cpu().numpy(), atol=2e-3)
    assert_lse_close(l2.cpu().numpy(), l1.cpu().numpy(), rtol=1e-4)


def test_window_rejects_pageable_host_memory():
    """A tail in ordinary (pageable) host memory is refused before any launch."""
    w = synth.WORKLOADS["decode-b8-kv256k-c65536"]
    inp = synth.make_inputs(w, B=1, N=200, q0=199)
    cfg = cfg_for(w, to_dev(inp["freq_factors"]))
    k = torch.from_numpy(inp["k"].view(np.int16)).view(torch.bfloat16)
    rt = dca.Region(dca.KV_BF16, k[:, 100:].contiguous())          # plain CPU tensor
    with pytest.raises(dca.DcaError) as e:
        dca.attention_window(cfg, to_dev(inp["q"]), to_dev(inp["q_pos"]),
                             dca.Region(dca.KV_BF16, k[:, :100].contiguous().to(dev())), rt)
    assert e.value.status == dca.ERR_INVALID_ARGUMENT
