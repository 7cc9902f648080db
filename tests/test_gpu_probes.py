"""Sensitive parity at the real workload shapes: the distance and needle probes of tests/probes.py on
the 4k, 32k and 1M-slice prefills and the 256k-key decode (bf16, q8_0 and q4_0 caches), through the
entry points and launch configurations the benchmark times, against the fp64 oracle on sampled rows.

Each probe first asserts that it bites (the oracle's O is large where the probe says it must be),
then holds the GPU to the usual bar: max|d| <= 1e-2, ||d||/||O|| <= 1e-2 per (row, head), LSE within
1e-3 relative.  For the distance probe the per-row relative error is also taken over the
non-rotary dims alone, because the rotary dims of every key (the values, K = V) are one constant
vector whose norm would otherwise hide an error in which keys win.  The distance probe's scores
spread about ALPHA * scale = 8.5 (a query of rotary norm ALPHA against keys of unit RMS), not 1: its
LSE is held to 1e-3 of max(8.5, |lse|), since fp16 rotated operands move a score by a fixed fraction
of that spread whatever value the LSE itself takes.
"""
import numpy as np
import pytest
import torch

import oracle
import probes
from dual_chunk_attention_amd import dca, synth
from gpu_util import assert_lse_close, assert_o_close, cfg_for, rows_of, sample_rows, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (label, workload); each runs the distance probe, then the needle probe
    ("prefill-4k", "prefill-4k-c1024"),
    ("prefill-32k", "prefill-32k-c8192"),
    ("decode-256k", "decode-b8-kv256k-c65536"),
    ("decode-256k-q8", "decode-b8-kv256k-c65536-q8"),
    ("decode-256k-q4", "decode-b8-kv256k-c65536-q4"),
    ("prefill-1m-slice", "prefill-4k-at-1m-c65536"),
]
PARAMS = [(label, name, kind) for label, name in CASES for kind in ("distance", "needle")]

_BASE = {}


def _base_inputs(name):
    """The workload's seeded inputs, drawn once per workload (the two probes modify copies)."""
    if name not in _BASE:
        _BASE.clear()
        _BASE[name] = synth.make_inputs(name)
    src = _BASE[name]
    return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in src.items()}


def _rows(w):
    if w.T == 1:
        return rows_of(w.B, 1, [(b, 0) for b in range(w.B)])
    if w.q0 > 0:   # the 1M slice: every row costs about 1M keys x 16 heads in the oracle
        extra = np.random.default_rng(17).integers(0, w.T, 3).tolist()
        return rows_of(1, w.T, [(0, t) for t in sorted({0, 1, w.T // 2 - 1, w.T - 2, w.T - 1, *extra})])
    return rows_of(1, w.T, sample_rows(w.T, w.chunk, 24, seed=w.seed + 100))


def _run(inp, w):
    ffd = to_dev(inp["freq_factors"])
    cfg = cfg_for(w, ffd)
    q, qp = to_dev(inp["q"]), to_dev(inp["q_pos"])
    if w.dtype == "bf16":
        o, lse = dca.attention(cfg, q, qp, to_dev(inp["k"]), o_dtype=torch.bfloat16)
    else:
        codes = torch.from_numpy(inp["k_codes"]).to("cuda:0")
        scales = torch.from_numpy(inp["k_scales"].view(np.int16)).to("cuda:0")
        fn = dca.attention_q8 if w.dtype == "q8_0" else dca.attention_q4
        o, lse = fn(cfg, q, qp, codes, scales, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().reshape(w.B * w.T, w.Hq, w.D), lse.cpu().numpy().reshape(w.B * w.T, w.Hq)


def _oracle(inp, w, rows):
    kw = dict(chunk=w.chunk, n_rot=w.n_rot, theta=w.theta, scale=w.scale,
              freq_factors=inp["freq_factors"].astype(np.float64), rows=rows, per_regime=False)
    if w.dtype == "bf16":
        return oracle.attention(inp["q"], inp["q_pos"], inp["k"], **kw)
    fn = oracle.attention_q8 if w.dtype == "q8_0" else oracle.attention_q4
    return fn(inp["q"], inp["q_pos"], inp["k_codes"], inp["k_scales"], **kw)


@pytest.mark.parametrize("label,name,kind", PARAMS, ids=[f"{p[0]}-{p[2]}" for p in PARAMS])
def test_probe_at_workload_shape(label, name, kind):
    inp = _base_inputs(name)
    w = inp["w"]
    rows = _rows(w)
    print(f"probe {kind} on {name}: {rows.size} rows", flush=True)
    R = w.n_rot
    if kind == "distance":
        probes.distance_probe(inp)
    else:
        _, _, bounds, st = oracle.remap(w.chunk, inp["q_pos"], w.N)
        assert st == 0
        planted = probes.needle_probe(inp, bounds, rows)
        assert planted
    got_o, got_l = _run(inp, w)
    res = _oracle(inp, w, rows)
    want_o, want_l = res["o"], res["lse"]
    sel = res["rows"]
    # the probe bites: large outputs where it says so
    assert np.abs(want_o).max() > 0.3
    if kind == "distance":
        tail = np.sqrt((want_o[..., R:] ** 2).sum(-1))
        assert np.median(tail) > 0.25, np.median(tail)
    else:
        pos = {x: i for i, x in enumerate(sel.tolist())}
        norms = [np.linalg.norm(want_o[pos[x], h]) for x, h, _, _ in planted]
        assert np.mean(np.array(norms) > 5.0) > 0.8, np.percentile(norms, [5, 50, 95])
    assert_o_close(got_o[sel], want_o)
    if kind == "distance":
        assert_o_close(got_o[sel][..., R:], want_o[..., R:], what="O (non-rotary dims)")
    floor = probes.ALPHA * w.scale if kind == "distance" else 1.0
    assert_lse_close(got_l[sel], want_l, floor=floor)
