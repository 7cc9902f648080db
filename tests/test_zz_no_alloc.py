"""dca_attention_noalloc (the entry point for callers that cannot allocate) through the C ABI: its
output equals dca_attention's, bit for bit, on two calls in a row on one GPU, the second with a
smaller input (the static scratch keeps the first call's contents), and both lie within the parity
bar of the fp64 oracle; calls whose workspace exceeds the static scratch are refused before any
launch."""
import numpy as np
import pytest
import torch

import oracle
from dual_chunk_attention_amd import dca, synth
from gpu_util import assert_lse_close, assert_o_close, cfg_for, rows_of, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (label, [(B, T, N, q0, chunk), ...] called in this order)
    ("decode", [(4, 1, 100000, 99999, 16384), (2, 1, 30000, 29999, 16384)]),
    ("prefill", [(1, 1024, 1024, 0, 256), (1, 300, 700, 400, 128)]),
    ("decode-then-prefill", [(8, 1, 120000, 119999, 32768), (1, 200, 200, 0, 64)]),
]


def _one(B, T, N, q0, chunk, seed):
    w = synth.Workload("noalloc", B, T, q0, N, chunk, 16, 2, "bf16", seed)
    inp = synth.make_inputs(w)
    cfg = cfg_for(w, to_dev(inp["freq_factors"]))
    q, qp, k = to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"])
    ref_o, ref_l = dca.attention(cfg, q, qp, k, o_dtype=torch.float32)
    out = torch.empty((B, T, 16, 512), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, T, 16), dtype=torch.float32, device="cuda:0")
    return w, inp, cfg, (q, qp, k), (ref_o, ref_l), (out, lse)


@pytest.mark.parametrize("label,calls", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry_point(label, calls):
    runs = [_one(*c, seed=200 + i) for i, c in enumerate(calls)]
    torch.cuda.synchronize()
    for w, inp, cfg, args, ref, outs in runs:   # back to back on the current stream
        dca.attention_noalloc(cfg, *args, *outs)
    torch.cuda.synchronize()
    for w, inp, cfg, args, (ref_o, ref_l), (o, l) in runs:
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
        B, T = w.B, w.T
        rows = rows_of(B, T, [(b, t) for b in range(B) for t in sorted({0, T // 2, T - 1})])
        res = oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=w.chunk, n_rot=w.n_rot,
                               theta=w.theta, scale=w.scale, freq_factors=inp["freq_factors"].astype(np.float64),
                               rows=rows, per_regime=False)
        assert_o_close(o.cpu().numpy().reshape(B * T, 16, 512)[rows], res["o"])
        assert_lse_close(l.cpu().numpy().reshape(B * T, 16)[rows], res["lse"])


def test_noalloc_refuses_workspace_beyond_the_static_scratch():
    cfg = dca.Config(chunk=8192)
    c = cfg.c()
    need = dca.lib().dca_attention_workspace_size(c, dca.BF16, 1, 32768, 32768)
    assert need > dca.NOALLOC_SCRATCH_BYTES
    vp = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    st = dca.lib().dca_attention_noalloc(c, dca.BF16, 1, 32768, vp.data_ptr(), vp.data_ptr(), vp.data_ptr(),
                                         32768, dca.BF16, vp.data_ptr(), vp.data_ptr(), None)
    assert st == dca.ERR_UNSUPPORTED
    assert b"static scratch" in dca.lib().dca_last_error()
