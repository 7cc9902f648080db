"""GPU parity of the decode over a q8_0 or q4_0 key cache (dca_attention_q8 / dca_attention_q4)
against the fp64 oracle reading the same codes and scales.

Bar as for the bf16 path: O within 1e-2 absolute, LSE within 1e-3 relative, an all-empty row
exactly (0, -inf).  The kernel forms each key value d*q in fp16 (one rounding) and the rotated dims
in fp16, as the bf16 path does; the oracle is exact fp64.
"""
import numpy as np
import pytest
import torch

import oracle
from dual_chunk_attention_amd import dca, synth
from gpu_util import assert_lse_close, assert_o_close, cfg_for, dev, to_dev

pytestmark = pytest.mark.gpu

# format -> (full workload, GPU entry point, oracle, block store, dtype name)
FORMATS = {
    "q8": ("decode-b8-kv256k-c65536-q8", dca.attention_q8, oracle.attention_q8, synth.q8_0_blocks, "q8_0"),
    "q4": ("decode-b8-kv256k-c65536-q4", dca.attention_q4, oracle.attention_q4, synth.q4_0_blocks, "q4_0"),
}
FMTS = list(FORMATS)


def _dev_cache(inp):
    codes = torch.from_numpy(np.ascontiguousarray(inp["k_codes"])).to(dev())
    scales = torch.from_numpy(np.ascontiguousarray(inp["k_scales"]).view(np.int16)).to(dev())
    return codes, scales


def _run_and_check(fmt, inp, w, chunk=None, remap_mode=0, o_dtype=torch.float32, rows=None):
    _, gpu_fn, oracle_fn, _, _ = FORMATS[fmt]
    B, T, Hq, D = inp["q"].shape
    ffd = to_dev(inp["freq_factors"]) if w.ff_uniform else None
    cfg = cfg_for(w, ffd, chunk=chunk, remap_mode=remap_mode)
    codes, scales = _dev_cache(inp)
    o, lse = gpu_fn(cfg, to_dev(inp["q"]), to_dev(inp["q_pos"]), codes, scales, o_dtype=o_dtype)
    torch.cuda.synchronize()
    ff = inp["freq_factors"].astype(np.float64) if w.ff_uniform else None
    res = oracle_fn(inp["q"], inp["q_pos"], inp["k_codes"], inp["k_scales"],
                    chunk=w.chunk if chunk is None else chunk, n_rot=w.n_rot, theta=w.theta,
                    scale=w.scale, freq_factors=ff, rows=rows, per_regime=False, remap_mode=remap_mode)
    sel = res["rows"]
    got_o = o.float().cpu().numpy().reshape(B * T, Hq, D)[sel]
    got_l = lse.cpu().numpy().reshape(B * T, Hq)[sel]
    assert_o_close(got_o, res["o"])
    assert_lse_close(got_l, res["lse"])
    empty = np.isneginf(res["lse"])
    assert (got_o[empty] == 0).all()
    return res


CASES = [
    # (label, overrides, chunk, remap mode)
    ("kv20k-c4096", dict(B=2, N=20000, q0=19999), 4096, 0),
    ("t3-c3000", dict(B=2, T=3, N=9000, q0=8000), 3000, 0),       # c not a multiple of 64
    ("t8-tiny-ragged", dict(B=1, T=8, N=70, q0=62), 16, 0),        # one partial tile, all regimes
    ("t64-split", dict(B=1, T=64, N=600, q0=536), 128, 0),         # T past the bf16 decode cut
    ("single-key", dict(B=1, T=1, N=1, q0=0), 64, 0),
    ("empty-cache", dict(B=2, T=2, N=0, q0=0), 64, 0),
    ("page-c", dict(B=2, N=20000, q0=19999), 4096, dca.REMAP_PAGE_C),
    ("page-2c", dict(B=1, T=2, N=9000, q0=8998), 3000, dca.REMAP_PAGE_2C),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("label,over,chunk,mode", CASES, ids=[c[0] for c in CASES])
def test_quant_decode_cases(label, over, chunk, mode, fmt):
    inp = synth.make_inputs(FORMATS[fmt][0], **over)
    res = _run_and_check(fmt, inp, inp["w"], chunk=chunk, remap_mode=mode)
    if label == "empty-cache":
        assert np.isneginf(res["lse"]).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_quant_decode_full_workload(fmt):
    """The 256k-key, batch-8 decode over the quantized cache at its real sizes and chunk, bf16
    output as timed; every head of three of the eight rows (the oracle's cost is ~256k keys per
    row)."""
    inp = synth.make_inputs(FORMATS[fmt][0])
    _run_and_check(fmt, inp, inp["w"], o_dtype=torch.bfloat16, rows=np.array([0, 5, 7], np.int64))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (8, 2), (16, 1)])
def test_quant_gqa_ratios(Hq, Hkv, fmt):
    w = synth.Workload("gqa-" + fmt, 2, 2, 3000, 3002, 1024, Hq, Hkv, FORMATS[fmt][4], 79)
    _run_and_check(fmt, synth.make_inputs(w), w)


def _needle_inputs(fmt, T, N, q0, seed, scale_q=1.0):
    """Float keys with needles (a few keys set to the unit-RMS direction of a query head's tail),
    then stored in the quantized format: the needles dominate their row's softmax, so |O| ~ 1 and
    the 1e-2 bar bites.  scale_q > 1 makes the needle scores far exceed everything before them
    (rescale path)."""
    w = synth.Workload("needle-" + fmt, 1, T, q0, N, 256 if T > 1 else 1024, 16, 2, FORMATS[fmt][4], seed)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(seed + 1)
    q = synth.bf16_to_f32(inp["q"]).copy()
    k = rng.standard_normal((1, N, 2, 512)).astype(np.float32)
    for t in range(T):
        i = q0 + t
        q[0, t, :, 128:] *= scale_q
        for j, h in [(i - (t % 3), 3), (max(0, i - 300 - t), 11), (int(rng.integers(0, i + 1)), 6)]:
            qq = q[0, t, h, 128:]
            k[0, j, h // 8, 128:] = qq / np.sqrt(np.mean(qq ** 2))
    inp["q"] = synth.bf16_bits(q)
    inp["k_codes"], inp["k_scales"] = FORMATS[fmt][3](k)
    return inp, w


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,N,q0,scale_q", [(1, 3000, 2999, 1.0), (4, 5000, 4990, 1.0),
                                             (1, 3000, 2999, 12.0)])
def test_quant_needles(T, N, q0, scale_q, fmt):
    inp, w = _needle_inputs(fmt, T, N, q0, 41 + T, scale_q)
    res = _run_and_check(fmt, inp, w)
    assert np.abs(res["o"]).max() > 0.3
    if scale_q > 1:
        assert res["lse"].max() > 100.0


@pytest.mark.parametrize("fmt", FMTS)
def test_quant_bitwise_deterministic(fmt):
    inp = synth.make_inputs(FORMATS[fmt][0], B=2, N=50000, q0=49999)
    w = inp["w"]
    cfg = cfg_for(w, to_dev(inp["freq_factors"]), chunk=8192)
    codes, scales = _dev_cache(inp)
    q, qp = to_dev(inp["q"]), to_dev(inp["q_pos"])
    gpu_fn = FORMATS[fmt][1]
    o1, l1 = gpu_fn(cfg, q, qp, codes, scales)
    o2, l2 = gpu_fn(cfg, q, qp, codes, scales)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("fmt", FMTS)
def test_quant_magnitude_factor(fmt):
    """rope_attn_factor = 0.7 through the quantized decode (the factor rides on the cos/sin tables)."""
    inp = synth.make_inputs(FORMATS[fmt][0], B=2, N=9000, q0=8999)
    w = inp["w"]
    B, T, Hq, D = inp["q"].shape
    cfg = cfg_for(w, to_dev(inp["freq_factors"]), chunk=4096)
    cfg.rope_attn_factor = 0.7
    codes, scales = _dev_cache(inp)
    o, lse = FORMATS[fmt][1](cfg, to_dev(inp["q"]), to_dev(inp["q_pos"]), codes, scales, o_dtype=torch.float32)
    torch.cuda.synchronize()
    res = FORMATS[fmt][2](inp["q"], inp["q_pos"], inp["k_codes"], inp["k_scales"], chunk=4096, n_rot=w.n_rot,
                          theta=w.theta, scale=w.scale, freq_factors=inp["freq_factors"].astype(np.float64),
                          per_regime=False, attn_factor=0.7)
    assert_o_close(o.cpu().numpy().reshape(B * T, Hq, D), res["o"])
    assert_lse_close(lse.cpu().numpy().reshape(B * T, Hq), res["lse"])
