"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle on the same seeded inputs.

Integer outputs (positions, intervals) must match bit-exactly; O within 1e-2 absolute and LSE within
1e-3 relative (see gpu_util).  Large workloads are checked on stratified sampled rows (every chunk's
local offsets 0, 1, c/2, c-2, c-1, plus random rows); small ones on every row.
"""
import numpy as np
import pytest
import torch

import oracle
from dual_chunk_attention_amd import dca, synth
from gpu_util import (assert_lse_close, assert_o_close, cfg_for, dev, rows_of, sample_rows, to_dev)

pytestmark = pytest.mark.gpu


def _inputs(w, **kw):
    inp = synth.make_inputs(w, **kw)
    w = inp["w"]
    ff = to_dev(inp["freq_factors"]) if w.ff_uniform else None
    return inp, w, ff


def _oracle_attention(inp, w, rows=None, chunk=None, per_regime=True, round_rotated_bf16=False,
                      remap_mode=0):
    ff = inp["freq_factors"].astype(np.float64) if w.ff_uniform else None
    return oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=w.chunk if chunk is None else chunk,
                            n_rot=w.n_rot, theta=w.theta, scale=w.scale, freq_factors=ff, rows=rows,
                            per_regime=per_regime, round_rotated_bf16=round_rotated_bf16,
                            remap_mode=remap_mode)


# ----------------------------------------------------------------------------------------------
# a1: remap, bit-exact
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_remap_bit_exact_on_workloads(name):
    w = synth.WORKLOADS[name]
    q_pos = (w.q0 + np.arange(w.T, dtype=np.int64)).astype(np.int32)
    q_pos = np.ascontiguousarray(np.broadcast_to(q_pos, (w.B, w.T)))
    pos_q, pos_k, bounds = dca.remap_positions(cfg_for(w), to_dev(q_pos), w.N)
    torch.cuda.synchronize()
    o_pq, o_pk, o_b, st = oracle.remap(w.chunk, q_pos, w.N)
    assert st == 0
    assert np.array_equal(pos_q.cpu().numpy().reshape(3, -1), o_pq)
    assert np.array_equal(pos_k.cpu().numpy(), o_pk)
    assert np.array_equal(bounds.cpu().numpy().reshape(3, -1, 2), o_b)


@pytest.mark.parametrize("c,n_kv", [(1, 50), (7, 100), (64, 64), (1000, 300), (5, 0)])
def test_remap_bit_exact_edge_positions(c, n_kv):
    q_pos = np.array([[-5, -1, 0, 1, 6, 7, 8, 49, 63, 64, 99, 100, 299, 300, 1 << 30]], np.int32)
    cfg = dca.Config(chunk=c)
    pos_q, pos_k, bounds = dca.remap_positions(cfg, to_dev(q_pos), n_kv)
    torch.cuda.synchronize()
    o_pq, o_pk, o_b, st = oracle.remap(c, q_pos, n_kv)
    assert np.array_equal(pos_q.cpu().numpy().reshape(3, -1), o_pq)
    assert np.array_equal(pos_k.cpu().numpy(), o_pk)
    assert np.array_equal(bounds.cpu().numpy().reshape(3, -1, 2), o_b)


PAGE_MODES = [dca.REMAP_PAGE_C, dca.REMAP_PAGE_2C]


@pytest.mark.parametrize("mode", PAGE_MODES)
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_remap_page_modes_bit_exact_on_workloads(name, mode):
    w = synth.WORKLOADS[name]
    q_pos = (w.q0 + np.arange(w.T, dtype=np.int64)).astype(np.int32)
    q_pos = np.ascontiguousarray(np.broadcast_to(q_pos, (w.B, w.T)))
    pos_q, pos_k, bounds = dca.remap_positions(cfg_for(w, remap_mode=mode), to_dev(q_pos), w.N)
    torch.cuda.synchronize()
    o_pq, o_pk, o_b, st = oracle.remap(w.chunk, q_pos, w.N, mode=mode)
    assert st == 0
    assert np.array_equal(pos_q.cpu().numpy().reshape(3, -1), o_pq)
    assert np.array_equal(pos_k.cpu().numpy(), o_pk)
    assert np.array_equal(bounds.cpu().numpy().reshape(3, -1, 2), o_b)


@pytest.mark.parametrize("mode", PAGE_MODES)
@pytest.mark.parametrize("c,n_kv", [(1, 50), (7, 100), (64, 64), (1000, 300), (5, 0)])
def test_remap_page_modes_edge_positions(c, n_kv, mode):
    q_pos = np.array([[-5, -1, 0, 1, 6, 7, 8, 49, 63, 64, 99, 100, 299, 300, 1 << 29]], np.int32)
    cfg = dca.Config(chunk=c, remap_mode=mode)
    pos_q, pos_k, bounds = dca.remap_positions(cfg, to_dev(q_pos), n_kv)
    torch.cuda.synchronize()
    o_pq, o_pk, o_b, st = oracle.remap(c, q_pos, n_kv, mode=mode)
    assert np.array_equal(pos_q.cpu().numpy().reshape(3, -1), o_pq)
    assert np.array_equal(pos_k.cpu().numpy(), o_pk)
    assert np.array_equal(bounds.cpu().numpy().reshape(3, -1, 2), o_b)


# ----------------------------------------------------------------------------------------------
# a2: partial RoPE
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("inplace", [False, True])
def test_rope_partial(bf16, inplace):
    rng = np.random.default_rng(5)
    rows, H, D, n_rot = 96, 16, 512, 128
    x32 = rng.standard_normal((rows, H, D)).astype(np.float32)
    pos = np.concatenate([[0, 1, 2, 8191, 8192, 65535, 131071, 1048575, (1 << 31) - 1],
                          rng.integers(0, 1 << 21, rows - 9)]).astype(np.int32)
    ff = rng.uniform(1, 8, n_rot // 2).astype(np.float32)
    if bf16:
        xb = synth.bf16_bits(x32)
        x_ref = synth.bf16_to_f32(xb).astype(np.float64)
        xd = to_dev(xb)
    else:
        x_ref = x32.astype(np.float64)
        xd = to_dev(x32)
    cfg = dca.Config(head_dim=D, n_rot=n_rot, n_head_q=H, n_head_kv=H, freq_factors=to_dev(ff))
    x_in = xd.clone()
    y = dca.rope_partial(cfg, x_in, to_dev(pos), out=x_in if inplace else None)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    want = oracle.rope(x_ref, pos, n_rot, 1.0e6, ff.astype(np.float64))
    # dims >= n_rot: bit-exact copy
    assert np.array_equal(got[..., n_rot:], x_ref[..., n_rot:])
    # rotated dims: fp32 rotation of fp64 angles, then (bf16) round to nearest
    err = np.abs(got[..., :n_rot] - want[..., :n_rot])
    mag = np.abs(x_ref[..., :n_rot // 2]) + np.abs(x_ref[..., n_rot // 2:n_rot])
    mag = np.concatenate([mag, mag], axis=-1)
    bound = (2.0 ** -8 * np.abs(want[..., :n_rot]) if bf16 else 0.0) + 2e-6 * mag + 1e-30
    assert (err <= bound).all(), float((err / bound).max())


# ----------------------------------------------------------------------------------------------
# a5: N-way LSE merge
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n_parts", [1, 2, 3, 8])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_lse_merge(n_parts, out_bf16):
    rng = np.random.default_rng(n_parts)
    rows, D = 1000, 512
    o = rng.standard_normal((n_parts, rows, D)).astype(np.float32)
    l = (rng.standard_normal((n_parts, rows)) * 5).astype(np.float32)
    l[:, :7] = -np.inf                                  # all parts empty
    l[rng.random((n_parts, rows)) < 0.3] = -np.inf      # some parts empty
    o[np.isneginf(l)] = np.nan                          # an empty part's O must never be read
    got_o, got_l = dca.lse_merge([to_dev(o[p]) for p in range(n_parts)], [to_dev(l[p]) for p in range(n_parts)],
                                 torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    want_o, want_l = oracle.merge(np.nan_to_num(o.astype(np.float64)), l.astype(np.float64))
    g = got_o.float().cpu().numpy()
    tol = 2.0 ** -8 * np.abs(want_o) + 1e-5 if out_bf16 else 1e-5
    assert np.isfinite(g).all()
    assert (np.abs(g - want_o) <= tol).all()
    assert_lse_close(got_l.cpu().numpy(), want_l, rtol=1e-6)
    assert (g[:7] == 0).all() and np.isneginf(got_l.cpu().numpy()[:7]).all()


# ----------------------------------------------------------------------------------------------
# a3/a4: one regime pass at a time, against the oracle's per-regime partials
# ----------------------------------------------------------------------------------------------

REGIME_CASES = [
    # (label, workload name, overrides, chunk override, rows sampled (None = all))
    ("fp32-tiny", "prefill-256-c64-fp32", {}, None, None),
    ("bf16-prefill-ragged", "prefill-4k-c1024", dict(T=300, N=300), 64, None),
    ("bf16-prefill-offset", "prefill-4k-c1024", dict(T=200, q0=700, N=1000), 128, None),
    ("bf16-decode", "decode-b8-kv256k-c65536", dict(B=2, N=20000, q0=19999), 4096, None),
    ("bf16-decode-midchunk", "decode-b8-kv256k-c65536", dict(B=2, T=3, N=9000, q0=8000), 3000, None),
]


@pytest.mark.parametrize("label,name,over,chunk,rows", REGIME_CASES, ids=[c[0] for c in REGIME_CASES])
def test_attn_regime_each_regime(label, name, over, chunk, rows):
    inp, w, ffd = _inputs(name, **over)
    B, T = inp["q"].shape[:2]
    N = inp["k"].shape[1]
    cfg = cfg_for(w, ffd, chunk=chunk)
    c = cfg.chunk
    q, k, qp = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["q_pos"])
    pos_q, pos_k, bounds = dca.remap_positions(cfg, qp, N)
    k_rot = dca.rope_partial(cfg, k.reshape(B * N, w.Hkv, w.D), pos_k.repeat(B)).reshape(k.shape)
    k_rot = k_rot[..., :w.n_rot].contiguous()   # the entry point takes the rotary dims only
    # this entry point receives rotated operands in the data type (bf16 here): the oracle rounds
    # its own fp64 rotations the same way, so the comparison isolates the attention pass
    res = _oracle_attention(inp, w, chunk=c, round_rotated_bf16=w.dtype == "bf16")
    for r in range(3):
        q_r = dca.rope_partial(cfg, q.reshape(B * T, w.Hq, w.D), pos_q[r].reshape(-1).contiguous())
        o_r, l_r = dca.attn_regime(cfg, r, q_r.reshape(q.shape), bounds, k_rot, k)
        torch.cuda.synchronize()
        want_o = res["o_reg"][r].reshape(B, T, w.Hq, w.D)
        want_l = res["lse_reg"][r].reshape(B, T, w.Hq)
        assert_o_close(o_r.cpu().numpy(), want_o, atol=1e-4 if w.dtype == "f32" else 1e-2, what=f"O_{r}")
        assert_lse_close(l_r.cpu().numpy(), want_l, rtol=1e-5 if w.dtype == "f32" else 1e-3, what=f"lse_{r}")
        # an empty regime is exactly (0, -inf)
        empty = np.isneginf(want_l)
        assert (o_r.cpu().numpy()[empty] == 0).all()


# ----------------------------------------------------------------------------------------------
# the whole path: dca_attention on every workload
# ----------------------------------------------------------------------------------------------

E2E = [
    ("prefill-256-c64-fp32", None, torch.float32),
    ("prefill-4k-c1024", 96, torch.bfloat16),
    ("prefill-32k-c8192", 48, torch.bfloat16),
    ("decode-b8-kv256k-c65536", 0, torch.bfloat16),
    ("prefill-4k-at-1m-c65536", 4, torch.bfloat16),
]


@pytest.mark.parametrize("name,n_random,o_dtype", E2E, ids=[e[0] for e in E2E])
def test_attention_end_to_end(name, n_random, o_dtype):
    inp, w, ffd = _inputs(name)
    B, T = w.B, w.T
    if n_random is None:
        rows = None
    elif w.T == 1:
        rows = rows_of(B, T, [(b, 0) for b in range(B)])
    elif w.q0 > 0:   # slice: few rows (each costs ~1M keys in the oracle)
        rows = rows_of(B, T, [(0, 0), (0, 1), (0, 2047), (0, 4094), (0, 4095)] +
                       [(0, int(t)) for t in np.random.default_rng(9).integers(0, T, n_random)])
    else:
        rows = rows_of(B, T, sample_rows(T, w.chunk, n_random, seed=w.seed))
    q, k, qp = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["q_pos"])
    o, lse = dca.attention(cfg_for(w, ffd), q, qp, k, o_dtype=o_dtype)
    torch.cuda.synchronize()
    res = _oracle_attention(inp, w, rows=rows, per_regime=False)
    sel = res["rows"]
    got_o = o.float().cpu().numpy().reshape(B * T, w.Hq, w.D)[sel]
    got_l = lse.cpu().numpy().reshape(B * T, w.Hq)[sel]
    assert_o_close(got_o, res["o"], atol=1e-4 if w.dtype == "f32" else 1e-2)
    assert_lse_close(got_l, res["lse"], rtol=1e-5 if w.dtype == "f32" else 1e-3)


PAGE_E2E = [
    ("prefill-256-c64-fp32", None, torch.float32),
    ("prefill-4k-c1024", 32, torch.bfloat16),
    ("decode-b8-kv256k-c65536", 0, torch.bfloat16),
]


@pytest.mark.parametrize("mode", PAGE_MODES)
@pytest.mark.parametrize("name,n_random,o_dtype", PAGE_E2E, ids=[e[0] for e in PAGE_E2E])
def test_attention_page_modes(name, n_random, o_dtype, mode):
    """dca_attention under the page-literal remap tables (succ = the whole previous chunk; inter
    query at c or 2c): the decode row now has a non-empty succ regime of c keys."""
    inp, w, ffd = _inputs(name)
    B, T = w.B, w.T
    if n_random is None:
        rows = None
    elif w.T == 1:
        rows = rows_of(B, T, [(b, 0) for b in range(B)])
    else:
        rows = rows_of(B, T, sample_rows(T, w.chunk, n_random, seed=w.seed + mode))
    q, k, qp = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["q_pos"])
    o, lse = dca.attention(cfg_for(w, ffd, remap_mode=mode), q, qp, k, o_dtype=o_dtype)
    torch.cuda.synchronize()
    res = _oracle_attention(inp, w, rows=rows, per_regime=False, remap_mode=mode)
    sel = res["rows"]
    got_o = o.float().cpu().numpy().reshape(B * T, w.Hq, w.D)[sel]
    got_l = lse.cpu().numpy().reshape(B * T, w.Hq)[sel]
    assert_o_close(got_o, res["o"], atol=1e-4 if w.dtype == "f32" else 1e-2)
    assert_lse_close(got_l, res["lse"], rtol=1e-5 if w.dtype == "f32" else 1e-3)


# ----------------------------------------------------------------------------------------------
# structured probes (random inputs make |O| ~ N^-1/2, too small for a 1e-2 bound to bite)
# ----------------------------------------------------------------------------------------------

def _probe_inputs(T, N, q0, seed, kind):
    w = synth.Workload("probe", 1, T, q0, N, 256, 16, 2, "bf16", seed)
    inp = synth.make_inputs(w)
    q = synth.bf16_to_f32(inp["q"]).copy()
    k = synth.bf16_to_f32(inp["k"]).copy()
    rng = np.random.default_rng(seed + 1)
    if kind == "distance":
        # q: rotary part a unit vector in pair 0 scaled by 6, tail zero; k: rotary part the
        # orthogonal unit vector of pair 0 (so s = scale*6*sin(d w_0)), tail random.
        q[..., :] = 0.0
        q[..., 0] = 6.0 * np.sqrt(512)
        k[..., :128] = 0.0
        k[..., 64] = 1.0
    else:  # needles: a few keys equal to the direction of a query's tail (unit RMS)
        for t in rng.integers(0, T, 24):
            i = q0 + t
            for j in {int(i), int(max(0, i - 3)), int(max(0, i - 300)), int(rng.integers(0, i + 1))}:
                for g in range(2):
                    qq = q[0, t, 8 * g + int(rng.integers(0, 8)), 128:]
                    k[0, j, g, 128:] = qq / np.sqrt(np.mean(qq ** 2))   # unit RMS, like every key
    inp["q"], inp["k"] = synth.bf16_bits(q), synth.bf16_bits(k)
    return inp, w


@pytest.mark.parametrize("kind", ["distance", "needles"])
@pytest.mark.parametrize("T,N,q0", [(1024, 1024, 0), (1, 3000, 2999), (256, 2000, 1744)])
def test_structured_probes(kind, T, N, q0):
    inp, w = _probe_inputs(T, N, q0, seed=31 + T, kind=kind)
    ffd = to_dev(inp["freq_factors"])
    cfg = cfg_for(w, ffd)
    o, lse = dca.attention(cfg, to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"]), o_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = None if T <= 256 else rows_of(1, T, sample_rows(T, w.chunk, 64, seed=3))
    res = _oracle_attention(inp, w, rows=rows, per_regime=False)
    sel = res["rows"]
    got_o = o.cpu().numpy().reshape(T, w.Hq, w.D)[sel]
    assert np.abs(res["o"]).max() > 0.3          # the probe really produces large outputs
    assert_o_close(got_o, res["o"])
    assert_lse_close(lse.cpu().numpy().reshape(T, w.Hq)[sel], res["lse"])


# ----------------------------------------------------------------------------------------------
# invariants across paths
# ----------------------------------------------------------------------------------------------

def test_chunk_covering_sequence_is_plain_attention():
    """c >= seqlen: every row is intra-only; succ/inter partials are exactly empty."""
    inp, w, ffd = _inputs("prefill-4k-c1024", T=512, N=512)
    cfg = cfg_for(w, ffd, chunk=4096)
    o, lse = dca.attention(cfg, to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"]), o_dtype=torch.float32)
    torch.cuda.synchronize()
    res = _oracle_attention(inp, w, chunk=4096, per_regime=True)
    assert np.isneginf(res["lse_reg"][1:]).all()
    assert_o_close(o.cpu().numpy().reshape(-1, w.Hq, w.D), res["o"])
    assert_lse_close(lse.cpu().numpy().reshape(-1, w.Hq), res["lse"])


def test_decode_row_matches_prefill_row():
    """The split-KV decode path at position p equals row p of the prefill path (both on GPU)."""
    inp, w, ffd = _inputs("prefill-4k-c1024", T=2048, N=2048)
    cfg = cfg_for(w, ffd, chunk=512)
    q, k = to_dev(inp["q"]), to_dev(inp["k"])
    o_pf, l_pf = dca.attention(cfg, q, to_dev(inp["q_pos"]), k, o_dtype=torch.float32)
    for p in [5, 511, 512, 1000, 2047]:
        qd = q[:, p:p + 1].contiguous()
        o_d, l_d = dca.attention(cfg, qd, to_dev(np.array([[p]], np.int32)), k, o_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_o_close(o_d.cpu().numpy()[0, 0], o_pf.cpu().numpy()[0, p], atol=5e-3)
        assert_lse_close(l_d.cpu().numpy()[0, 0], l_pf.cpu().numpy()[0, p], rtol=5e-4)


@pytest.mark.parametrize("shape", ["prefill", "decode"])
def test_bitwise_deterministic(shape):
    if shape == "prefill":
        inp, w, ffd = _inputs("prefill-4k-c1024", T=1024, N=1024)
        cfg = cfg_for(w, ffd, chunk=256)
    else:
        inp, w, ffd = _inputs("decode-b8-kv256k-c65536", B=2, N=50000, q0=49999)
        cfg = cfg_for(w, ffd, chunk=8192)
    q, k, qp = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["q_pos"])
    o1, l1 = dca.attention(cfg, q, qp, k)
    o2, l2 = dca.attention(cfg, q, qp, k)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (8, 2), (16, 1)])
def test_gqa_ratios_bf16(Hq, Hkv):
    w = synth.Workload("gqa", 1, 160, 0, 160, 48, Hq, Hkv, "bf16", 77)
    inp = synth.make_inputs(w)
    ffd = to_dev(inp["freq_factors"])
    o, lse = dca.attention(cfg_for(w, ffd), to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"]),
                           o_dtype=torch.float32)
    torch.cuda.synchronize()
    res = _oracle_attention(inp, w, per_regime=False)
    assert_o_close(o.cpu().numpy().reshape(-1, Hq, 512), res["o"])
    assert_lse_close(lse.cpu().numpy().reshape(-1, Hq), res["lse"])


def test_batch_of_prefill_sequences():
    w = synth.Workload("b3", 3, 130, 0, 130, 40, 16, 2, "bf16", 78)
    inp = synth.make_inputs(w)
    ffd = to_dev(inp["freq_factors"])
    o, lse = dca.attention(cfg_for(w, ffd), to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"]),
                           o_dtype=torch.float32)
    torch.cuda.synchronize()
    res = _oracle_attention(inp, w, per_regime=False)
    assert_o_close(o.cpu().numpy().reshape(-1, 16, 512), res["o"])
    assert_lse_close(lse.cpu().numpy().reshape(-1, 16), res["lse"])


@pytest.mark.parametrize("T,N,q0,factor,lse_min", [(256, 256, 0, 12.0, 100.0), (1, 3000, 2999, 12.0, 100.0),
                                                    (256, 256, 0, 3.4, 50.0), (256, 256, 0, 4.5, 70.0)],
                         ids=["prefill-x12", "decode-x12", "prefill-x3.4", "prefill-x4.5"])
def test_reference_move_with_extreme_scores(T, N, q0, factor, lse_min):
    """Queries scaled by `factor` aligned with unit-RMS needle keys, so that the needle scores
    exceed everything seen before.  x12: by far more than 128 (log2 units): the prefill kernel's
    exponents overflow to inf, its end-of-pass check of the row sums catches it and the workgroup
    runs its sequence again against the exact row maxima; the decode kernel rescales.  x3.4: by
    about 70: the sums stay below 2^80 and the first pass's result is kept.  x4.5: by about 95:
    finite exponents whose sums pass 2^80, so the sequence runs again.  Values stay unit RMS, so
    the 1e-2 bar applies; LSE is checked at 1e-3."""
    w = synth.Workload("extreme", 1, T, q0, N, 64 if T > 1 else 1024, 16, 2, "bf16", 91)
    inp = synth.make_inputs(w)
    q = synth.bf16_to_f32(inp["q"]).copy()
    k = synth.bf16_to_f32(inp["k"]).copy()
    rng = np.random.default_rng(92)
    rows = [T - 1] if T == 1 else list(range(3, T, 7))      # distinct positions, distinct keys
    for t in rows:
        i = q0 + int(t)
        for h in range(16):
            q[0, t, h, 128:] *= factor
        # a later (closer) key aligned with head 3's query, an earlier one with head 11's
        for j, h in [(i - (t % 3), 3), (max(0, i - 5 - (t % 3)), 11)]:
            qq = q[0, t, h, 128:]
            k[0, j, h // 8, 128:] = qq / np.sqrt(np.mean(qq ** 2))
    inp["q"], inp["k"] = synth.bf16_bits(q), synth.bf16_bits(k)
    ffd = to_dev(inp["freq_factors"])
    o, lse = dca.attention(cfg_for(w, ffd), to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"]),
                           o_dtype=torch.float32)
    torch.cuda.synchronize()
    res = _oracle_attention(inp, w, per_regime=False)
    assert res["lse"].max() > lse_min            # the needle scores are as large as intended
    assert_o_close(o.cpu().numpy().reshape(-1, 16, 512), res["o"])
    assert_lse_close(lse.cpu().numpy().reshape(-1, 16), res["lse"])


# ----------------------------------------------------------------------------------------------
# YaRN magnitude factor on the rotated dims
# ----------------------------------------------------------------------------------------------

MAG_CASES = [
    ("fp32-tiny", "prefill-256-c64-fp32", {}, None, torch.float32),
    ("bf16-prefill", "prefill-4k-c1024", dict(T=640, N=640), 256, torch.float32),
    ("bf16-decode", "decode-b8-kv256k-c65536", dict(B=2, N=20000, q0=19999), 4096, torch.float32),
]


@pytest.mark.parametrize("label,name,over,chunk,o_dtype", MAG_CASES, ids=[c[0] for c in MAG_CASES])
def test_attention_magnitude_factor(label, name, over, chunk, o_dtype):
    """rope_attn_factor = 1.6 on every path of dca_attention against the oracle with the same
    factor (the rotary part of each score scales by 2.56)."""
    inp, w, ffd = _inputs(name, **over)
    mag = 1.6
    cfg = cfg_for(w, ffd, chunk=chunk)
    cfg.rope_attn_factor = mag
    o, lse = dca.attention(cfg, to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"]), o_dtype=o_dtype)
    torch.cuda.synchronize()
    ff = inp["freq_factors"].astype(np.float64) if w.ff_uniform else None
    B, T = inp["q"].shape[:2]
    res = oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=cfg.chunk, n_rot=w.n_rot, theta=w.theta,
                           scale=w.scale, freq_factors=ff, per_regime=False, attn_factor=mag)
    tol_o, tol_l = (1e-4, 1e-5) if w.dtype == "f32" else (1e-2, 1e-3)
    assert_o_close(o.float().cpu().numpy().reshape(B * T, w.Hq, w.D), res["o"], atol=tol_o)
    assert_lse_close(lse.cpu().numpy().reshape(B * T, w.Hq), res["lse"], rtol=tol_l)
    plain = oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=cfg.chunk, n_rot=w.n_rot, theta=w.theta,
                             scale=w.scale, freq_factors=ff, per_regime=False, rows=[0])
    assert np.abs(plain["lse"] - res["lse"][:1]).max() > 1e-3      # the factor is not a no-op here


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (16, 2), (16, 1)])
def test_gqa_ratios_decode_bf16(Hq, Hkv):
    """The split-KV decode with G = Hq/Hkv query heads per KV head (the 16 MFMA columns padded)."""
    w = synth.Workload("gqa-dec", 2, 2, 2998, 3000, 1024, Hq, Hkv, "bf16", 81)
    inp = synth.make_inputs(w)
    ffd = to_dev(inp["freq_factors"])
    o, lse = dca.attention(cfg_for(w, ffd), to_dev(inp["q"]), to_dev(inp["q_pos"]), to_dev(inp["k"]),
                           o_dtype=torch.float32)
    torch.cuda.synchronize()
    res = _oracle_attention(inp, w, per_regime=False)
    assert_o_close(o.cpu().numpy().reshape(-1, Hq, 512), res["o"])
    assert_lse_close(lse.cpu().numpy().reshape(-1, Hq), res["lse"])


def test_concurrent_streams_with_own_workspaces():
    """Calls on two streams at once, each with its own workspace, give the results of calls made one
    after the other (the library keeps no state between calls)."""
    inp_p, wp, ffp = _inputs("prefill-4k-c1024", T=1024, N=1024)
    inp_d, wd, ffdd = _inputs("decode-b8-kv256k-c65536", B=2, N=30000, q0=29999)
    cfg_p, cfg_d = cfg_for(wp, ffp, chunk=256), cfg_for(wd, ffdd, chunk=8192)
    args_p = (to_dev(inp_p["q"]), to_dev(inp_p["q_pos"]), to_dev(inp_p["k"]))
    args_d = (to_dev(inp_d["q"]), to_dev(inp_d["q_pos"]), to_dev(inp_d["k"]))
    o_p1, l_p1 = dca.attention(cfg_p, *args_p)
    o_d1, l_d1 = dca.attention(cfg_d, *args_d)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            op, lp = dca.attention(cfg_p, *args_p)
        with torch.cuda.stream(s2):
            od, ld = dca.attention(cfg_d, *args_d)
        outs.append((op, lp, od, ld))
    torch.cuda.synchronize()
    for op, lp, od, ld in outs:
        assert torch.equal(op.view(torch.int16), o_p1.view(torch.int16)) and torch.equal(lp, l_p1)
        assert torch.equal(od.view(torch.int16), o_d1.view(torch.int16)) and torch.equal(ld, l_d1)
