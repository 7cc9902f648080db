"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and the parity bar.

Parity bar: integer outputs bit-exact; O within 1e-2 absolute; LSE within 1e-3 relative
(|d lse| <= 1e-3 * max(1, |lse|), a floor so that rows whose LSE is near 0 are held to 1e-3
absolute); an empty regime must be exactly (0, -inf).

Per-row relative error.  With i.i.d. unit-RMS queries and keys at scale 1/sqrt(512) the scores have
unit spread, attention is nearly uniform, and |O| per element falls like (e/N)^(1/2): about 0.009
at 32k keys, 0.003 at 256k, 0.0016 at 1M.  The absolute bound alone then passes an all-zero O.
So every end-to-end comparison also bounds, for each (row, head), the relative error
||O_gpu - O_oracle||_2 / ||O_oracle||_2 by O_RTOL = 1e-2.  Derivation: the softmax weights enter the
value product rounded to bf16 (relative error <= 2^-9 each, independent across keys), and the
output is rounded to bf16 once more (<= 2^-9 per element); independent roundings of size u give a
relative error of about u/sqrt(3) ~ 1.1e-3 each in the 2-norm, whatever the number of keys, and
the fp16 rotated operands move each score by well under 1e-3 (relative weight error of the same
size).  1e-2 leaves a margin of about 5x over their sum, while a dropped span of keys, a wrong
rotation or a missing regime moves the ratio by 0.1 to 1.
"""
import numpy as np
import torch

from dual_chunk_attention_amd import dca, synth

O_ATOL = 1e-2
O_RTOL = 1e-2
LSE_RTOL = 1e-3


def dev():
    return torch.device("cuda:0")


def to_dev(arr):
    """uint16 bf16 bits -> bf16 tensor; float32 -> fp32 tensor; int32 -> int32."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev())


def cfg_for(w, ff_dev=None, chunk=None, remap_mode=0):
    return dca.Config(head_dim=w.D, n_rot=w.n_rot, n_head_q=w.Hq, n_head_kv=w.Hkv,
                      chunk=w.chunk if chunk is None else chunk, rope_theta=w.theta, scale=w.scale,
                      freq_factors=ff_dev, remap_mode=remap_mode)


def row_rel_err(got, want):
    """||got - want||_2 / ||want||_2 over the last axis (one value per (row, head)); rows whose
    reference is exactly 0 (empty) give 0 if got is 0 there too, else inf."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    dn = np.sqrt(((got - want) ** 2).sum(axis=-1))
    wn = np.sqrt((want ** 2).sum(axis=-1))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(wn > 0, dn / np.where(wn > 0, wn, 1.0), np.where(dn > 0, np.inf, 0.0))
    return rel


def assert_o_close(got, want, atol=O_ATOL, rtol=O_RTOL, what="O"):
    """max|d| <= atol over all elements and ||d||/||O|| <= rtol per (row, head); the message gives
    both.  Returns (max|d|, max relative row error)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - want)
    i = np.unravel_index(np.argmax(err), err.shape)
    rel = row_rel_err(got, want)
    ri = np.unravel_index(np.argmax(rel), rel.shape) if rel.size else ()
    msg = (f"{what}: max|d| {err.max():.3e} at {i} (got {got[i]}, want {want[i]}); "
           f"max ||d||/||O|| {rel.max() if rel.size else 0.0:.3e} at row {ri}; max|O| {np.abs(want).max():.3e}")
    assert err.max() <= atol, msg
    assert rel.size == 0 or rel.max() <= rtol, msg
    return float(err.max()), float(rel.max()) if rel.size else 0.0


def assert_lse_close(got, want, rtol=LSE_RTOL, what="lse", floor=1.0):
    """|d lse| <= rtol * max(floor, |lse|).  The floor is the spread of the scores the LSE is made
    of (1 for unit-RMS queries and keys at scale 1/sqrt(D)): an LSE near 0 only means that the
    scores happen to cancel, and its error is that of the scores, whose size the spread sets."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    inf_w = np.isneginf(want)
    assert (np.isneginf(got) == inf_w).all(), f"{what}: -inf pattern differs"
    g, w_ = got[~inf_w], want[~inf_w]
    if g.size == 0:
        return 0.0
    err = np.abs(g - w_) / np.maximum(floor, np.abs(w_))
    i = int(np.argmax(err))
    assert err.max() <= rtol, f"{what}: max rel err {err.max():.3e} (got {g[i]}, want {w_[i]}, floor {floor})"
    return float(err.max())


def rows_of(B, T, picks):
    """Flat row indices b*T + t for a list of (b, t)."""
    return np.array([b * T + t for b, t in picks], np.int64)


def sample_rows(T, c, n_random, seed, B=1):
    """Stratified query rows: every chunk's local offsets {0, 1, c/2, c-2, c-1} plus random ones,
    plus the first and last rows."""
    rng = np.random.default_rng(seed)
    ts = {0, T - 1}
    for ch in range(0, T, c):
        for off in (0, 1, c // 2, c - 2, c - 1):
            if 0 <= ch + off < T:
                ts.add(ch + off)
    ts.update(rng.integers(0, T, n_random).tolist())
    picks = [(b, t) for b in range(B) for t in sorted(ts)]
    return picks
