"""GPU parity of dca_attention (bf16) at the edges of its cases: one key per chunk, a chunk that
no tile size divides, the query count on either side of the cut between the split-KV decode pass
(T <= 8) and the single prefill pass, a cache with no cells, a single key, and a short prefill
continuing a longer cache.  Bar as in the other parity tests: O within 1e-2 absolute, LSE within
1e-3 relative, and a row without keys exactly (0, -inf).
"""
import numpy as np
import pytest
import torch

import oracle
from dual_chunk_attention_amd import dca, synth
from gpu_util import assert_lse_close, assert_o_close, cfg_for, to_dev

pytestmark = pytest.mark.gpu

EDGES = [
    # (label, B, T, N, q0, chunk)
    ("c1-prefill", 1, 40, 40, 0, 1),            # every key its own chunk
    ("c1-decode", 2, 1, 100, 99, 1),
    ("c2-prefill-offset", 1, 24, 90, 66, 2),
    ("t9-prefill-cut", 1, 9, 9, 0, 4),          # the fewest queries the prefill pass serves
    ("t8-decode-cut", 1, 8, 500, 492, 100),     # the most queries the split-KV pass serves
    ("c33-prefill", 1, 130, 130, 0, 33),        # chunk edges inside key tiles and query blocks
    ("c33-decode", 2, 1, 700, 699, 33),
    ("t17-offset-ragged", 1, 17, 300, 283, 64),
    ("single-key-decode", 1, 1, 1, 0, 64),
    ("c-over-cache-prefill", 1, 12, 12, 0, 1000),   # c larger than the cache
    ("empty-cache-prefill", 1, 20, 0, 0, 16),
    ("empty-cache-decode", 2, 1, 0, 0, 16),
]


@pytest.mark.parametrize("label,B,T,N,q0,chunk", EDGES, ids=[e[0] for e in EDGES])
def test_attention_edges(label, B, T, N, q0, chunk):
    w = synth.Workload("edge-" + label, B, T, q0, N, chunk, 16, 2, "bf16", 101)
    inp = synth.make_inputs(w)
    ffd = to_dev(inp["freq_factors"])
    o, lse = dca.attention(cfg_for(w, ffd), to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"]),
                           o_dtype=torch.float32)
    torch.cuda.synchronize()
    res = oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=chunk, n_rot=w.n_rot, theta=w.theta,
                           scale=w.scale, freq_factors=inp["freq_factors"].astype(np.float64),
                           per_regime=False)
    got_o = o.cpu().numpy().reshape(B * T, w.Hq, w.D)
    got_l = lse.cpu().numpy().reshape(B * T, w.Hq)
    assert_o_close(got_o, res["o"])
    assert_lse_close(got_l, res["lse"])
    empty = np.isneginf(res["lse"])
    assert (got_o[empty] == 0).all()
    if N == 0:
        assert empty.all()
