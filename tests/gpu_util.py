"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and the parity bar.

Parity bar (the benchmark spec's tolerance, restated): integer outputs bit-exact; O within 1e-2 absolute;
LSE within 1e-3 relative (|d lse| <= 1e-3 * max(1, |lse|), a floor so that rows whose LSE is near 0
are held to 1e-3 absolute); an empty regime must be exactly (0, -inf).
"""
import numpy as np
import torch

from dual_chunk_attention_amd import dca, synth

O_ATOL = 1e-2
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


def assert_o_close(got, want, atol=O_ATOL, what="O"):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - want)
    i = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= atol, f"{what}: max|d| {err.max():.3e} at {i} (got {got[i]}, want {want[i]})"
    return float(err.max())


def assert_lse_close(got, want, rtol=LSE_RTOL, what="lse"):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    inf_w = np.isneginf(want)
    assert (np.isneginf(got) == inf_w).all(), f"{what}: -inf pattern differs"
    g, w_ = got[~inf_w], want[~inf_w]
    if g.size == 0:
        return 0.0
    err = np.abs(g - w_) / np.maximum(1.0, np.abs(w_))
    assert err.max() <= rtol, f"{what}: max rel err {err.max():.3e}"
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
