"""Pins of the CPU oracle against facts the pages and mathematics fix (CPU only).

Every check here compares the oracle with something other than itself: a hand-derived table,
an invariant the pages state, a closed form, a textbook or library routine, or an independent
dense (materialised) formulation on tiny inputs.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from dual_chunk_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------------
# remap
# ----------------------------------------------------------------------------------------------

def _load_golden_remap():
    rows = []
    with open(os.path.join(GOLDEN, "remap_c4.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, c = line.split("|")
            i, n_kv = map(int, a.split())
            pq = list(map(int, b.split()))
            bd = list(map(int, c.split()))
            rows.append((i, n_kv, pq, bd))
    return rows


@pytest.mark.parametrize("case", _load_golden_remap(), ids=lambda c: f"i{c[0]}_n{c[1]}")
def test_remap_golden_table(case):
    i, n_kv, pq, bd = case
    pos_q, pos_k, bounds, st = oracle.remap(4, [i], n_kv)
    assert st == 0
    assert pos_q[:, 0].tolist() == pq
    assert bounds[:, 0, :].reshape(-1).tolist() == bd
    assert pos_k.tolist() == [j % 4 for j in range(n_kv)]


def _load_golden_remap_page():
    rows = []
    with open(os.path.join(GOLDEN, "remap_c4_page.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, c = line.split("|")
            mode, i, n_kv = map(int, a.split())
            rows.append((mode, i, n_kv, list(map(int, b.split())), list(map(int, c.split()))))
    return rows


@pytest.mark.parametrize("case", _load_golden_remap_page(), ids=lambda c: f"m{c[0]}_i{c[1]}_n{c[2]}")
def test_remap_golden_table_page_modes(case):
    mode, i, n_kv, pq, bd = case
    pos_q, pos_k, bounds, st = oracle.remap(4, [i], n_kv, mode=mode)
    assert st == 0
    assert pos_q[:, 0].tolist() == pq
    assert bounds[:, 0, :].reshape(-1).tolist() == bd
    assert pos_k.tolist() == [j % 4 for j in range(n_kv)]


@pytest.mark.parametrize("mode", [oracle.REMAP_PAGE_C, oracle.REMAP_PAGE_2C])
@pytest.mark.parametrize("c", [1, 2, 3, 4, 7, 16])
def test_remap_page_modes_partition_and_distances(c, mode):
    """Page-literal tables ("Section C design"): regimes by chunk index alone, still a partition
    of the causal keys; intra and succ see the true distance (succ up to 2c - 1), inter sees
    P_inter - (j mod c) with P_inter = c (distances [1, c]) or 2c (distances [c + 1, 2c])."""
    n_kv = 90
    qpos = np.arange(0, n_kv + 6, dtype=np.int32)
    pos_q, pos_k, bounds, st = oracle.remap(c, qpos, n_kv, mode=mode)
    assert st == 0
    p_inter = c if mode == oracle.REMAP_PAGE_C else 2 * c
    for row, i in enumerate(qpos):
        seen = np.zeros(n_kv, np.int32)
        for r in range(3):
            lo, hi = bounds[r, row]
            if hi < lo:
                assert (lo, hi) == (0, -1)
                continue
            seen[lo:hi + 1] += 1
            for j in range(lo, hi + 1):
                assert oracle.regime(i, j, c, n_kv, mode) == r
                chunk_gap = i // c - j // c
                assert chunk_gap == r if r != oracle.INTER else chunk_gap >= 2
                d = int(pos_q[r, row]) - int(pos_k[j])
                if r == oracle.INTER:
                    assert pos_q[r, row] == p_inter and d == p_inter - j % c
                else:
                    assert d == i - j and 0 <= d < 2 * c
        upto = min(int(i), n_kv - 1)
        assert (seen[: upto + 1] == 1).all() and (seen[upto + 1:] == 0).all()


@pytest.mark.parametrize("c", [1, 2, 3, 4, 7, 16, 64])
def test_remap_partition_and_distances(c):
    """The three regimes partition the causal keys (DCA feature page, "Section C design") and
    every remapped rotary distance lies in [0, c); intra and succ see the true distance."""
    n_kv = 150
    qpos = np.arange(0, n_kv + 6, dtype=np.int32)
    pos_q, pos_k, bounds, st = oracle.remap(c, qpos, n_kv)
    assert st == 0
    for row, i in enumerate(qpos):
        seen = np.zeros(n_kv, np.int32)
        for r in range(3):
            lo, hi = bounds[r, row]
            if hi < lo:
                assert (lo, hi) == (0, -1)
                continue
            seen[lo:hi + 1] += 1
            for j in range(lo, hi + 1):
                assert oracle.regime(i, j, c, n_kv) == r
                d = int(pos_q[r, row]) - int(pos_k[j])
                assert 0 <= d < c, (i, j, r, d)
                if r != oracle.INTER:
                    assert d == i - j
        upto = min(int(i), n_kv - 1)
        assert (seen[: upto + 1] == 1).all() and (seen[upto + 1:] == 0).all()


def test_remap_empty_regimes():
    c, n_kv = 8, 64
    qpos = np.arange(n_kv, dtype=np.int32)
    _, _, bounds, _ = oracle.remap(c, qpos, n_kv)
    for i in qpos:
        succ_empty = bounds[1, i, 1] < bounds[1, i, 0]
        inter_empty = bounds[2, i, 1] < bounds[2, i, 0]
        assert succ_empty == (i < c or i % c == c - 1)
        assert inter_empty == (i < c)
        assert bounds[0, i, 1] >= bounds[0, i, 0]  # intra holds the diagonal


def test_remap_chunk_covers_sequence_is_plain_causal():
    """c >= seqlen: every key is intra at its true position (DCA feature page, flags section:
    DCA is inert when the chunk covers the sequence)."""
    n_kv = 97
    qpos = np.arange(n_kv, dtype=np.int32)
    pos_q, pos_k, bounds, _ = oracle.remap(128, qpos, n_kv)
    assert (pos_q[0] == qpos).all() and (pos_k == np.arange(n_kv)).all()
    assert (bounds[0, :, 0] == 0).all() and (bounds[0, :, 1] == qpos).all()
    assert (bounds[1:, :, 1] == -1).all()


# ----------------------------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------------------------

def _rope_complex(x, pos, n_rot, theta, ff):
    """Textbook RoPE as complex multiplication of (x_f + i x_{f+half}) by exp(i p w_f)."""
    half = n_rot // 2
    w = theta ** (-2.0 * np.arange(half) / n_rot) / ff
    z = x[..., :half] + 1j * x[..., half:n_rot]
    z = z * np.exp(1j * np.asarray(pos, np.float64)[:, None, None] * w)
    y = x.copy()
    y[..., :half] = z.real
    y[..., half:n_rot] = z.imag
    return y


def test_rope_closed_forms():
    rng = np.random.default_rng(11)
    rows, H, D, n_rot, theta = 9, 3, 40, 16, 1.0e6
    ff = rng.uniform(1, 8, n_rot // 2)
    x = rng.standard_normal((rows, H, D))
    pos = np.array([0, 1, 2, 5, 63, 64, 1000, 131071, 1048575])
    y = oracle.rope(x, pos, n_rot, theta, ff)
    # p = 0 is the identity, dims >= n_rot are copied
    assert np.array_equal(y[0], x[0])
    assert np.array_equal(y[..., n_rot:], x[..., n_rot:])
    # pair norms are preserved
    half = n_rot // 2
    n0 = x[..., :half] ** 2 + x[..., half:n_rot] ** 2
    n1 = y[..., :half] ** 2 + y[..., half:n_rot] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # the complex-exponential form of rotary embedding (freq_factors divide the frequency)
    np.testing.assert_allclose(y, _rope_complex(x, pos, n_rot, theta, ff), rtol=0, atol=1e-11)
    # unit vector e_0: (cos(p w_0), sin(p w_0)) with w_0 = 1 / ff[0]
    e0 = np.zeros((1, 1, D))
    e0[0, 0, 0] = 1.0
    for p in [1, 7, 65535]:
        yy = oracle.rope(e0, [p], n_rot, theta, ff)
        assert yy[0, 0, 0] == pytest.approx(math.cos(p / ff[0]), abs=1e-10)  # angle rounding ~ p*2^-52
        assert yy[0, 0, half] == pytest.approx(math.sin(p / ff[0]), abs=1e-10)


def test_rope_composition_and_relative_invariance():
    rng = np.random.default_rng(12)
    D, n_rot, theta = 32, 32, 1.0e4
    ff = rng.uniform(1, 8, n_rot // 2)
    x = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for a, b in [(3, 5), (100, 7), (4095, 4097)]:
        ab = oracle.rope(oracle.rope(x, [a], n_rot, theta, ff), [b], n_rot, theta, ff)
        np.testing.assert_allclose(ab, oracle.rope(x, [a + b], n_rot, theta, ff), atol=1e-10)
        for t in [1, 33, 1000]:
            s0 = np.sum(oracle.rope(x, [a], n_rot, theta, ff) * oracle.rope(k, [b], n_rot, theta, ff))
            s1 = np.sum(oracle.rope(x, [a + t], n_rot, theta, ff) * oracle.rope(k, [b + t], n_rot, theta, ff))
            assert s1 == pytest.approx(s0, abs=1e-9)


# ----------------------------------------------------------------------------------------------
# merge
# ----------------------------------------------------------------------------------------------

def test_merge_identity_and_empty_parts():
    rng = np.random.default_rng(13)
    rows, D = 5, 7
    o1 = rng.standard_normal((1, rows, D))
    l1 = rng.standard_normal((1, rows))
    o, l = oracle.merge(o1, l1)
    np.testing.assert_allclose(o, o1[0], rtol=1e-15)
    np.testing.assert_allclose(l, l1[0], rtol=1e-15)
    # a -inf part has weight 0 and its O (garbage here) is never used
    junk = np.full((1, rows, D), np.nan)
    o, l = oracle.merge(np.concatenate([o1, junk]), np.concatenate([l1, np.full((1, rows), -np.inf)]))
    np.testing.assert_allclose(o, o1[0], rtol=1e-15)
    # all parts empty -> O = 0, lse = -inf, no NaN
    o, l = oracle.merge(np.concatenate([junk, junk]), np.full((2, rows), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


def test_merge_equals_softmax_of_concatenation():
    """Merging per-part (O, lse) equals one softmax over the concatenated scores."""
    rng = np.random.default_rng(14)
    n, D = 50, 6
    s = rng.standard_normal(n) * 3
    v = rng.standard_normal((n, D))
    cuts = [0, 7, 8, 31, 50]
    o_parts, l_parts = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        lse = scipy.special.logsumexp(s[a:b])
        o_parts.append((np.exp(s[a:b] - lse)[:, None] * v[a:b]).sum(0)[None])
        l_parts.append([lse])
    o, l = oracle.merge(np.stack(o_parts), np.array(l_parts))
    p = scipy.special.softmax(s)
    np.testing.assert_allclose(o[0], p @ v, rtol=1e-12, atol=1e-14)
    assert l[0] == pytest.approx(scipy.special.logsumexp(s), rel=1e-14)


# ----------------------------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------------------------

def _small_inputs(B, T, N, Hq, Hkv, D, q0, seed, bf16=False):
    w = synth.Workload("t", B, T, q0, N, 4, Hq, Hkv, "bf16" if bf16 else "f32", seed, D=D,
                       n_rot=min(D, 16), ff_uniform=True)
    return synth.make_inputs(w)


def _eager_dca(q, qpos, k, c, n_rot, theta, scale, ff, mag=1.0):
    """Materialised DCA: three masked dense score blocks and one softmax (the eager form the
    DCA feature page rules out at scale, "Section-C VERDICT"), with complex-form RoPE; mag
    multiplies the rotated dims of q and k (YaRN magnitude)."""
    B, T, Hq, D = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    i = qpos.astype(np.int64)[:, :, None]                  # [B,T,1]
    j = np.arange(N, dtype=np.int64)[None, None, :]        # [1,1,N]
    ci, cj = np.floor_divide(i, c), np.floor_divide(j, c)
    causal = j <= i
    masks = [causal & (cj == ci), causal & (cj == ci - 1) & (i - j < c), causal & (i - j >= c)]
    qpos_r = [np.mod(qpos, c), np.mod(qpos, c) + c, np.full_like(qpos, c - 1)]
    kr = _rope_complex(k.reshape(B * N, Hkv, D), np.tile(np.arange(N) % c, B), n_rot, theta, ff)
    kr = kr.reshape(B, N, Hkv, D)
    kr[..., :n_rot] *= mag
    S = np.full((B, T, Hq, N), -np.inf)
    for r in range(3):
        qr = _rope_complex(q.reshape(B * T, Hq, D), qpos_r[r].reshape(-1), n_rot, theta, ff)
        qr = qr.reshape(B, T, Hq, D)
        qr[..., :n_rot] *= mag
        for h in range(Hq):
            s = scale * np.einsum("btd,bnd->btn", qr[:, :, h], kr[:, :, h // G])
            S[:, :, h, :] = np.where(masks[r], s, S[:, :, h, :])
    lse = scipy.special.logsumexp(S, axis=-1)
    P = np.exp(S - lse[..., None])
    P = np.nan_to_num(P)
    O = np.zeros((B, T, Hq, D))
    for h in range(Hq):
        O[:, :, h] = np.einsum("btn,bnd->btd", P[:, :, h], k[:, :, h // G])
    return O, lse


@pytest.mark.parametrize("B,T,N,Hq,Hkv,D,q0,c", [
    (1, 37, 37, 2, 1, 24, 0, 4),      # ragged: T not a multiple of c
    (2, 9, 30, 4, 2, 16, 21, 5),      # decode-like tail block, batch 2, GQA 2
    (1, 20, 20, 1, 1, 16, 0, 1),      # c = 1: every earlier key is inter
    (1, 12, 40, 2, 2, 32, 28, 8),     # query block late in the cache
])
def test_attention_matches_eager_dense_form(B, T, N, Hq, Hkv, D, q0, c):
    inp = _small_inputs(B, T, N, Hq, Hkv, D, q0, seed=100 + T)
    q, k, qpos, ff = inp["q"], inp["k"], inp["q_pos"], inp["freq_factors"].astype(np.float64)
    n_rot, theta, scale = min(D, 16), 1.0e6, 1 / math.sqrt(D)
    res = oracle.attention(q, qpos, k, chunk=c, n_rot=n_rot, theta=theta, scale=scale, freq_factors=ff)
    O, lse = _eager_dca(q.astype(np.float64), qpos, k.astype(np.float64), c, n_rot, theta, scale, ff)
    np.testing.assert_allclose(res["o"], O.reshape(B * T, Hq, D), rtol=0, atol=1e-11)
    np.testing.assert_allclose(res["lse"], lse.reshape(B * T, Hq), rtol=1e-12)
    # partition claim: the merge of the per-regime partials is the union softmax
    o_m, l_m = oracle.merge(res["o_reg"].reshape(3, -1, D), res["lse_reg"].reshape(3, -1))
    np.testing.assert_allclose(o_m, res["o"].reshape(-1, D), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_m, res["lse"].reshape(-1), rtol=1e-13)


def test_attention_bf16_rounded_rotations_match_eager_form():
    """The rounded-rotation option equals the dense form with rotated q/k rounded by PyTorch's
    float->bf16 conversion (nearest-even)."""
    B, T, N, Hq, Hkv, D, q0, c = 1, 29, 29, 2, 1, 16, 0, 4
    inp = _small_inputs(B, T, N, Hq, Hkv, D, q0, seed=55)
    q, k, qpos, ff = inp["q"], inp["k"], inp["q_pos"], inp["freq_factors"].astype(np.float64)
    n_rot, theta, scale = 16, 1.0e6, 0.25
    res = oracle.attention(q, qpos, k, chunk=c, n_rot=n_rot, theta=theta, scale=scale, freq_factors=ff,
                           round_rotated_bf16=True)

    def rnd(x):
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()

    qf, kf = q.astype(np.float64), k.astype(np.float64)
    G = Hq // Hkv
    i = qpos.astype(np.int64)[0]
    j = np.arange(N)
    S = np.full((T, Hq, N), -np.inf)
    kr = _rope_complex(kf[0], j % c, n_rot, theta, ff)
    kr[..., :n_rot] = rnd(kr[..., :n_rot])
    for r, pq in enumerate([i % c, i % c + c, np.full_like(i, c - 1)]):
        qr = _rope_complex(qf[0], pq, n_rot, theta, ff)
        qr[..., :n_rot] = rnd(qr[..., :n_rot])
        for t in range(T):
            for h in range(Hq):
                for jj in range(N):
                    if oracle.regime(i[t], jj, c, N) == r:
                        S[t, h, jj] = scale * float(qr[t, h] @ kr[jj, h // G])
    lse = scipy.special.logsumexp(S, axis=-1)
    O = np.einsum("thn,nhd->thd", np.exp(S - lse[..., None]), np.repeat(kf[0], G, axis=1))
    np.testing.assert_allclose(res["lse"], lse, rtol=1e-12)
    np.testing.assert_allclose(res["o"], O, atol=1e-12)
    # and the rounding matters at this size (it is not a no-op)
    ex = oracle.attention(q, qpos, k, chunk=c, n_rot=n_rot, theta=theta, scale=scale, freq_factors=ff)
    assert np.abs(ex["lse"] - res["lse"]).max() > 1e-6


def test_attention_chunk_covers_sequence_equals_sdpa():
    """c >= seqlen collapses DCA to plain causal attention with RoPE at the true positions
    (DCA feature page, flags section and "Section B (gemma4)"); checked against PyTorch's
    scaled_dot_product_attention in fp64 on the CPU."""
    T, Hq, Hkv, D, n_rot, theta = 48, 4, 2, 32, 16, 1.0e6
    inp = _small_inputs(1, T, T, Hq, Hkv, D, 0, seed=7)
    q, k, qpos, ff = inp["q"], inp["k"], inp["q_pos"], inp["freq_factors"].astype(np.float64)
    scale = 1 / math.sqrt(D)
    res = oracle.attention(q, qpos, k, chunk=T, n_rot=n_rot, theta=theta, scale=scale, freq_factors=ff)
    qr = _rope_complex(q[0].astype(np.float64), np.arange(T), n_rot, theta, ff)   # [T,Hq,D]
    kr = _rope_complex(k[0].astype(np.float64), np.arange(T), n_rot, theta, ff)   # [T,Hkv,D]
    G = Hq // Hkv
    Qt = torch.from_numpy(qr).permute(1, 0, 2)                                     # [Hq,T,D]
    Kt = torch.from_numpy(np.repeat(kr, G, axis=1)).permute(1, 0, 2).contiguous()
    Vt = torch.from_numpy(np.repeat(k[0].astype(np.float64), G, axis=1)).permute(1, 0, 2).contiguous()
    O = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=True, scale=scale)
    S = (Qt @ Kt.transpose(1, 2)) * scale
    S = S.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    L = torch.logsumexp(S, dim=-1)
    np.testing.assert_allclose(res["o"], O.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"], L.permute(1, 0).numpy(), rtol=1e-13)


def test_attention_single_key_row():
    """Position 0 attends only itself: O = k_0 (un-rotated), lse = scale <q, k_0>."""
    inp = _small_inputs(1, 3, 3, 2, 1, 16, 0, seed=8)
    q, k, qpos = inp["q"], inp["k"], inp["q_pos"]
    res = oracle.attention(q, qpos, k, chunk=2, n_rot=16, theta=1e6, scale=0.25,
                           freq_factors=inp["freq_factors"].astype(np.float64), rows=[0])
    for h in range(2):
        np.testing.assert_allclose(res["o"][0, h], k[0, 0, 0].astype(np.float64), rtol=1e-15)
        assert res["lse"][0, h] == pytest.approx(0.25 * float(np.dot(q[0, 0, h].astype(np.float64),
                                                                      k[0, 0, 0].astype(np.float64))), rel=1e-13)


@pytest.mark.parametrize("i,c,n_kv", [(37, 8, 38), (63, 16, 64), (40, 16, 41), (100, 7, 101)])
@pytest.mark.parametrize("mode", [oracle.REMAP_BASELINE, oracle.REMAP_PAGE_C, oracle.REMAP_PAGE_2C])
def test_attention_distance_probe(i, c, n_kv, mode):
    """Probe: q's rotary part is (1,0) in pair 0 and zero elsewhere, k's rotary part is (0,1) in
    pair 0, tails of q are zero.  Then s_j = scale * A * sin(d_j w_0) with d_j the remapped
    distance: i - j for intra and succ, c - 1 - (j mod c) for inter (page modes: succ is the whole
    previous chunk, inter at c - (j mod c) or 2c - (j mod c)).  O's rotary dims equal the
    un-rotated key value (0, 1) exactly because values are not rotated."""
    D, n_rot, half, A, scale = 16, 8, 4, 3.0, 0.5
    ff = np.array([1.7, 2.0, 3.0, 5.0])
    rng = np.random.default_rng(i)
    q = np.zeros((1, 1, 1, D), np.float32)
    q[0, 0, 0, 0] = A
    k = np.zeros((1, n_kv, 1, D), np.float32)
    k[0, :, 0, half] = 1.0
    k[0, :, 0, n_rot:] = rng.standard_normal((n_kv, D - n_rot)).astype(np.float32)
    res = oracle.attention(q, np.array([[i]], np.int32), k, chunk=c, n_rot=n_rot, theta=1e6,
                           scale=scale, freq_factors=ff, remap_mode=mode)
    j = np.arange(min(i, n_kv - 1) + 1)
    same = (j // c) == (i // c)
    if mode == oracle.REMAP_BASELINE:
        near = (i - j) < c
        d = np.where(same | near, i - j, c - 1 - (j % c))
    else:
        near = (j // c) == (i // c) - 1
        p_inter = c if mode == oracle.REMAP_PAGE_C else 2 * c
        d = np.where(same | near, i - j, p_inter - (j % c))
    s = scale * A * np.sin(d / ff[0])
    p = scipy.special.softmax(s)
    assert res["lse"][0, 0] == pytest.approx(scipy.special.logsumexp(s), rel=1e-13)
    np.testing.assert_allclose(res["o"][0, 0, n_rot:], p @ k[0, j, 0, n_rot:].astype(np.float64), atol=1e-13)
    assert res["o"][0, 0, half] == pytest.approx(1.0, abs=1e-14)
    assert abs(res["o"][0, 0, 0]) < 1e-14


def test_attention_needle():
    """A key equal to a scaled copy of the query's tail dominates the softmax."""
    inp = _small_inputs(1, 1, 64, 1, 1, 64, 63, seed=9)
    q, k = inp["q"].copy(), inp["k"].copy()
    n_rot = 16
    k[0, 17, 0, n_rot:] = 6.0 * q[0, 0, 0, n_rot:]
    k[0, 17, 0, :n_rot] = 0.0
    res = oracle.attention(q, np.array([[63]], np.int32), k, chunk=16, n_rot=n_rot, theta=1e6,
                           scale=1 / 8, freq_factors=inp["freq_factors"].astype(np.float64))
    np.testing.assert_allclose(res["o"][0, 0], k[0, 17, 0].astype(np.float64), atol=1e-6)


# ----------------------------------------------------------------------------------------------
# input generator
# ----------------------------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# ----------------------------------------------------------------------------------------------
# q8_0 key cache
# ----------------------------------------------------------------------------------------------

def test_half_matches_numpy_float16_on_every_bit_pattern():
    """The oracle's binary16 decoder against numpy's float16 on all 65536 patterns."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half(int(b)) for b in bits])
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert np.array_equal(got[~nan], want[~nan])
    # hand values: 1, the smallest subnormal, -2, the largest finite, -0
    assert [oracle.half(b) for b in (0x3C00, 0x0001, 0xC000, 0x7BFF)] == [1.0, 2.0 ** -24, -2.0, 65504.0]
    assert math.copysign(1.0, oracle.half(0x8000)) == -1.0


def test_dequant_q8_hand_example():
    """Two blocks of one row, worked by hand: block 0 has d = 0.5 (0x3800), block 1 d = -3 * 2^-24
    (a negative subnormal scale, 0x8003); each value is d times its code."""
    codes = np.zeros((1, 64), np.int8)
    codes[0, :6] = [-128, -1, 0, 1, 127, 5]
    codes[0, 32:35] = [3, -7, 100]
    codes[0, 63] = -2
    scales = np.array([[0x3800, 0x8003]], np.uint16)
    want = np.zeros((1, 64))
    want[0, :6] = [-64.0, -0.5, 0.0, 0.5, 63.5, 2.5]
    s1 = -3.0 * 2.0 ** -24
    want[0, 32:35] = [3 * s1, -7 * s1, 100 * s1]
    want[0, 63] = -2 * s1
    got = oracle.dequant_q8(codes, scales)
    assert np.array_equal(got, want)


def test_q8_quantizer_round_trip_bound():
    """The synthetic q8_0 store: codes in [-127, 127], every nonzero block reaches |code| = 127,
    and d*q is within d/2 (half a step) plus the fp16 rounding of d of the drawn value."""
    x = np.random.default_rng(12).standard_normal((50, 3, 96)).astype(np.float32) * 4
    x[0, 0, :32] = 0.0                       # an all-zero block
    x[1, 1, 32:64] = 1e-6                    # a constant block of a tiny value (subnormal scale)
    codes, scales = synth.q8_0_blocks(x)
    assert codes.shape == x.shape and scales.shape == (50, 3, 3)
    assert codes.min() >= -127 and codes.max() <= 127
    blk = np.abs(codes.reshape(50, 3, 3, 32)).max(axis=-1)
    nonzero = np.abs(x.reshape(50, 3, 3, 32)).max(axis=-1) > 0
    assert (blk[nonzero] == 127).all() and (blk[~nonzero] == 0).all()
    d_exact = np.abs(x.reshape(50, 3, 3, 32)).max(axis=-1).astype(np.float64) / 127
    deq = oracle.dequant_q8(codes, scales).reshape(50, 3, 3, 32)
    err = np.abs(deq - x.reshape(50, 3, 3, 32).astype(np.float64))
    d_store = scales.view(np.float16).astype(np.float64)
    bound = d_exact / 2 * (1 + 1e-6) + np.abs(d_store - d_exact) * 127 + 1e-30
    assert (err <= bound[..., None]).all()


def test_q8_generator_is_deterministic_and_blocks_agree():
    """The chunked, threaded store equals q8_0_blocks of the same draws, for any chunking."""
    shape = (2, 40, 2, 64)
    c1, s1 = synth._normal_q8(np.random.default_rng(4), shape, chunk_elems=1 << 10)
    c2, s2 = synth._normal_q8(np.random.default_rng(4), shape, chunk_elems=1 << 14)
    x = np.random.default_rng(4).standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    c3, s3 = synth.q8_0_blocks(x)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.array_equal(c1, c3) and np.array_equal(s1, s3)


@pytest.mark.parametrize("mode", [oracle.REMAP_BASELINE, oracle.REMAP_PAGE_C])
def test_attention_q8_equals_attention_over_the_dequantized_cache(mode):
    """A q8_0 value d*q (11-bit times 8-bit significand) is exact in float32, so attention over the
    q8_0 cache must equal, to the last bit, attention over the float32 cache of d*q with the bf16
    queries widened to float32."""
    w = synth.Workload("t8", 2, 9, 40, 49, 8, 4, 2, "q8_0", 21, D=64, n_rot=16)
    inp = synth.make_inputs(w)
    ff = inp["freq_factors"].astype(np.float64)
    kw = dict(chunk=w.chunk, n_rot=w.n_rot, theta=w.theta, scale=0.125, freq_factors=ff, remap_mode=mode)
    res = oracle.attention_q8(inp["q"], inp["q_pos"], inp["k_codes"], inp["k_scales"], **kw)
    kf = oracle.dequant_q8(inp["k_codes"], inp["k_scales"])
    assert np.array_equal(kf.astype(np.float32).astype(np.float64), kf)
    ref = oracle.attention(synth.bf16_to_f32(inp["q"]), inp["q_pos"], kf.astype(np.float32), **kw)
    for key in ("o", "lse", "o_reg", "lse_reg"):
        assert np.array_equal(res[key], ref[key]), key
    # the cache really is quantized: the unquantized draws (the stream after Q) give a nearby but
    # different answer
    rng = np.random.default_rng(w.seed)
    synth._normal(rng, inp["q"].shape, True)
    kx = rng.standard_normal(kf.size, dtype=np.float32).reshape(kf.shape)
    assert np.abs(kf - kx).max() <= np.abs(kx).max() / 127 / 2 * 1.01
    raw = oracle.attention(synth.bf16_to_f32(inp["q"]), inp["q_pos"], kx, **kw)
    assert 0 < np.abs(raw["lse"] - res["lse"]).max() < 0.05


def test_dequant_q4_hand_example():
    """One row of two q4_0 blocks worked by hand: dim 2j in the low nibble of byte j.  Block 0 has
    d = 0.5 (0x3800): byte 0 = 0xF0 gives dims 0, 1 = (0 - 8, 15 - 8) * 0.5 = (-4, 3.5); byte 1 =
    0x98 gives (8 - 8, 9 - 8) * 0.5 = (0, 0.5).  Block 1 has d = -2 (0xC000): byte 16 = 0x1E gives
    dims 32, 33 = (14 - 8, 1 - 8) * -2 = (-12, 14)."""
    codes = np.full((1, 32), 0x88, np.uint8)       # every other dim: code 8, value 0
    codes[0, 0], codes[0, 1], codes[0, 16] = 0xF0, 0x98, 0x1E
    scales = np.array([[0x3800, 0xC000]], np.uint16)
    want = np.zeros((1, 64))
    want[0, :4] = [-4.0, 3.5, 0.0, 0.5]
    want[0, 32:34] = [-12.0, 14.0]
    assert np.array_equal(oracle.dequant_q4(codes, scales), want)


def test_q4_quantizer_round_trip_bound():
    """The synthetic q4_0 store: codes in [1, 15], every nonzero block reaches |n - 8| = 7, an
    all-zero block stores code 8, and d*(n - 8) is within half a step (plus the fp16 rounding of
    d) of the drawn value."""
    x = np.random.default_rng(13).standard_normal((40, 2, 64)).astype(np.float32) * 3
    x[0, 0, :32] = 0.0
    codes, scales = synth.q4_0_blocks(x)
    assert codes.shape == (40, 2, 32) and scales.shape == (40, 2, 2)
    n = np.stack([codes & 15, codes >> 4], axis=-1).reshape(40, 2, 64).astype(np.int64)
    assert n.min() >= 0 and n.max() <= 15
    dev_ = np.abs(n - 8).reshape(40, 2, 2, 32).max(axis=-1)
    nonzero = np.abs(x.reshape(40, 2, 2, 32)).max(axis=-1) > 0
    assert (dev_[nonzero] == 7).all() and (dev_[~nonzero] == 0).all()
    d_exact = np.abs(x.reshape(40, 2, 2, 32)).max(axis=-1).astype(np.float64) / 7
    d_store = scales.view(np.float16).astype(np.float64)
    err = np.abs(oracle.dequant_q4(codes, scales).reshape(40, 2, 2, 32) - x.reshape(40, 2, 2, 32))
    bound = d_exact / 2 * (1 + 1e-6) + np.abs(d_store - d_exact) * 7 + 1e-30
    assert (err <= bound[..., None]).all()


def test_q4_generator_is_deterministic_and_blocks_agree():
    shape = (2, 40, 2, 64)
    c1, s1 = synth._normal_q4(np.random.default_rng(5), shape, chunk_elems=1 << 10)
    c2, s2 = synth._normal_q4(np.random.default_rng(5), shape, chunk_elems=1 << 14)
    x = np.random.default_rng(5).standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    c3, s3 = synth.q4_0_blocks(x)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.array_equal(c1, c3) and np.array_equal(s1, s3)


@pytest.mark.parametrize("mode", [oracle.REMAP_BASELINE, oracle.REMAP_PAGE_2C])
def test_attention_q4_equals_attention_over_the_dequantized_cache(mode):
    """d * (n - 8) (11-bit times 4-bit significand) is exact in float32, so attention over the q4_0
    cache must equal, to the last bit, attention over the float32 cache of those values."""
    w = synth.Workload("t4", 2, 7, 30, 37, 8, 4, 2, "q4_0", 22, D=64, n_rot=16)
    inp = synth.make_inputs(w)
    ff = inp["freq_factors"].astype(np.float64)
    kw = dict(chunk=w.chunk, n_rot=w.n_rot, theta=w.theta, scale=0.125, freq_factors=ff, remap_mode=mode)
    res = oracle.attention_q4(inp["q"], inp["q_pos"], inp["k_codes"], inp["k_scales"], **kw)
    kf = oracle.dequant_q4(inp["k_codes"], inp["k_scales"])
    assert np.array_equal(kf.astype(np.float32).astype(np.float64), kf)
    ref = oracle.attention(synth.bf16_to_f32(inp["q"]), inp["q_pos"], kf.astype(np.float32), **kw)
    for key in ("o", "lse", "o_reg", "lse_reg"):
        assert np.array_equal(res[key], ref[key]), key


# ----------------------------------------------------------------------------------------------
# YaRN magnitude factor
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("mag", [0.5, 1.0, 1.7])
def test_attention_magnitude_factor_matches_eager_form(mag):
    """The factor multiplies the rotated dims of q and k: the oracle equals the eager dense form
    with the complex-form rotations scaled by the factor, and the rope's rotated dims scale by it
    while the pass-through dims stay bit-exact."""
    B, T, N, Hq, Hkv, D, q0, c = 1, 21, 30, 4, 2, 32, 9, 6
    inp = _small_inputs(B, T, N, Hq, Hkv, D, q0, seed=300)
    q, k, qpos, ff = inp["q"], inp["k"], inp["q_pos"], inp["freq_factors"].astype(np.float64)
    n_rot, theta, scale = 16, 1.0e6, 0.2
    res = oracle.attention(q, qpos, k, chunk=c, n_rot=n_rot, theta=theta, scale=scale, freq_factors=ff,
                           attn_factor=mag)
    O, lse = _eager_dca(q.astype(np.float64), qpos, k.astype(np.float64), c, n_rot, theta, scale, ff, mag)
    np.testing.assert_allclose(res["o"], O.reshape(B * T, Hq, D), rtol=0, atol=1e-11)
    np.testing.assert_allclose(res["lse"], lse.reshape(B * T, Hq), rtol=1e-12)
    x = q[0].astype(np.float64)
    y1 = oracle.rope(x, np.arange(T) * 7, n_rot, theta, ff)
    ym = oracle.rope(x, np.arange(T) * 7, n_rot, theta, ff, attn_factor=mag)
    np.testing.assert_allclose(ym[..., :n_rot], mag * y1[..., :n_rot], rtol=1e-15, atol=1e-15)
    assert np.array_equal(ym[..., n_rot:], x[..., n_rot:])
    if mag != 1.0:   # the factor really changes the result
        ref = oracle.attention(q, qpos, k, chunk=c, n_rot=n_rot, theta=theta, scale=scale, freq_factors=ff)
        assert np.abs(ref["lse"] - res["lse"]).max() > 1e-3


def test_magnitude_factor_rejected_when_not_positive():
    inp = _small_inputs(1, 2, 2, 1, 1, 16, 0, seed=301)
    with pytest.raises(RuntimeError):
        oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=4, n_rot=16, theta=1e6, scale=0.25,
                         attn_factor=0.0)
