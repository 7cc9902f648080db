"""Structured probe inputs at the real workload shapes (input recipes only: no arithmetic of the
method lives here; the oracle computes what the outputs must be).

With i.i.d. unit-RMS queries and keys the attention is nearly uniform and |O| is of order N^-1/2,
so a wrong rotation, a lost span of keys or a missing regime barely moves O.  The two probes below
make O large and make it depend on exactly those things (DCA feature page, "DCA algorithm (global
layers only)" and "Section C design": each regime scores a key at a remapped rotary distance).

distance probe: every query head's rotary dims are one fixed random direction of norm ALPHA (all 64
  rotary pairs excited), the same for every row, and its other dims are 0; every key's rotary dims
  are one fixed random unit-RMS vector per KV head, and its other dims keep their random draws.  A
  score is then a function of the key's remapped rotary distance alone, with a spread of several
  units, so a few distances carry most of the weight and O is a few keys' random tails.  Rotating a
  key at the wrong position, or a query at the wrong regime position, changes which keys win.
needle probe: for each checked row and each regime that has keys for it, one key at a random place
  in that regime's interval has its non-rotary dims set to the unit-RMS direction of one query
  head's non-rotary dims (a different head per regime), so that head's softmax lands on that key
  (score about 17 against unit-spread scores).  A span of keys that is skipped, read at the wrong
  place, or merged with the wrong weight loses its needle.
"""
import numpy as np

from dual_chunk_attention_amd import synth

ALPHA = 192.0      # norm of the query's rotary part in the distance probe (score spread ~ 5-6)


def _rot_vectors(seed, Hq, Hkv, n_rot):
    rng = np.random.default_rng(seed)
    qv = rng.standard_normal((Hq, n_rot))
    qv *= ALPHA / np.linalg.norm(qv, axis=1, keepdims=True)
    kv = rng.standard_normal((Hkv, n_rot))
    kv /= np.sqrt(np.mean(kv ** 2, axis=1, keepdims=True))
    return qv.astype(np.float32), kv.astype(np.float32)


def distance_probe(inp, seed=1234):
    """Turn the inputs of a workload (as synth.make_inputs returns them; bf16, q8_0 or q4_0) into the
    distance probe, in place; returns inp."""
    w = inp["w"]
    R = w.n_rot
    qv, kv = _rot_vectors(seed, w.Hq, w.Hkv, R)
    q = inp["q"]
    q[...] = 0
    q[..., :R] = synth.bf16_bits(qv)[None, None]
    if w.dtype == "bf16":
        inp["k"][..., :R] = synth.bf16_bits(kv)[None, None]
    else:
        blocks = synth.q8_0_blocks if w.dtype == "q8_0" else synth.q4_0_blocks
        codes, scales = blocks(np.pad(kv, ((0, 0), (0, w.D - R))))
        per = 1 if w.dtype == "q8_0" else 2
        inp["k_codes"][..., :R // per] = codes[:, :R // per][None, None]
        inp["k_scales"][..., :R // 32] = scales[:, :R // 32][None, None]
    return inp


def needle_probe(inp, bounds, rows, seed=4321):
    """Plant needles for the flat query rows `rows` (b*T + t) in place, using the per-regime key
    intervals `bounds` [3, B*T, 2] (inclusive, lo > hi empty) that the oracle's remap gives; returns
    the list of (row, head, regime, key) planted."""
    w = inp["w"]
    R, T = w.n_rot, w.T
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(seed)
    planted = []
    qf = inp["q"]
    for x in rows:
        b, t = divmod(int(x), T)
        for r in range(3):
            lo, hi = int(bounds[r, x, 0]), int(bounds[r, x, 1])
            if lo > hi:
                continue
            j = int(rng.integers(lo, hi + 1))
            for g in range(w.Hkv):
                h = g * G + (3 * r + int(t)) % G
                tail = synth.bf16_to_f32(qf[b, t, h, R:]).astype(np.float64)
                tail = (tail / np.sqrt(np.mean(tail ** 2))).astype(np.float32)
                if w.dtype == "bf16":
                    inp["k"][b, j, g, R:] = synth.bf16_bits(tail)
                else:
                    blocks = synth.q8_0_blocks if w.dtype == "q8_0" else synth.q4_0_blocks
                    codes, scales = blocks(np.concatenate([np.zeros(R, np.float32), tail]))
                    per = 1 if w.dtype == "q8_0" else 2
                    inp["k_codes"][b, j, g, R // per:] = codes[R // per:]
                    inp["k_scales"][b, j, g, R // 32:] = scales[R // 32:]
                planted.append((int(x), h, r, j))
    return planted
