"""Benchmark of the Dual Chunk Attention hot path on one MI355X.

One step = one dca_attention call (remap, query rotation x3, key rotation, the three regime passes,
the N-way merge) on the 32k-token prefill workload (one global layer: 16 query heads, 2 KV heads,
head_dim 512, chunk 8192, bf16, inputs resident in HBM).  The 256k-KV decode workload (8 sequences,
chunk 65536) is timed as a second leg.  Prints one JSON line.

value: query tokens per second of the prefill workload.  roofline: the regime-pass kernel, timed
live with HIP events recorded by the library between its stages, against the bf16 MFMA peak
(prefill) and the HBM peak (decode leg).  cpu_baseline: the fp64 CPU oracle timed on a sample of
query rows of the same workload on the host cores.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E


class HipEvents:
    """hipEvent_t handles through libamdhip64 (the library records them on its own stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
            self.arr[i] = ev.value

    def sync(self, i):
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(self.arr[i])) == 0

    def ms(self, i, j):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.arr[i]),
                                            ctypes.c_void_p(self.arr[j])) == 0
        return float(out.value)


def measured_traffic(kernel_file):
    """HBM bytes per launch of a kernel, from the FETCH_SIZE/WRITE_SIZE counter passes recorded in
    profiles/traffic.json; None when the kernel source changed since the counters were taken."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[kernel_file]
        src = open(os.path.join(ROOT, "dual_chunk_attention_amd", "csrc", kernel_file), "rb").read()
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != rec.get("sha256_16"):
        return None
    return float(rec["bytes"])


def to_dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def algorithmic_work(w):
    """Prefill: 4*D*Hq FLOP per attended (query, key) pair (QK^T and PV, every pair once across
    the three regimes).  Decode: B*N*Hkv*D*2 bytes (the cache read once; K = V)."""
    i = w.q0 + np.arange(w.T, dtype=np.float64)
    pairs = float(np.minimum(i + 1, w.N).sum()) * w.B
    flops = 4.0 * w.D * w.Hq * pairs
    kv_bytes = float(w.B) * w.N * w.Hkv * w.D * 2
    return flops, kv_bytes


def time_leg(torch, dca, w, inp, steps, warmup):
    cfg = dca.Config(head_dim=w.D, n_rot=w.n_rot, n_head_q=w.Hq, n_head_kv=w.Hkv, chunk=w.chunk,
                     rope_theta=w.theta, scale=w.scale, freq_factors=to_dev(torch, inp["freq_factors"]))
    q, k, qp = to_dev(torch, inp["q"]), to_dev(torch, inp["k"]), to_dev(torch, inp["q_pos"])
    ws = torch.empty(dca.attention_workspace_size(cfg, q.dtype, w.B, w.T, w.N), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.T, w.Hq), dtype=torch.float32, device="cuda:0")
    for _ in range(warmup):
        dca.attention(cfg, q, qp, k, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    ev = HipEvents(6 * steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(steps):
        sub = (ctypes.c_void_p * 6)(*ev.arr[6 * s:6 * s + 6])
        dca.set_stage_events(sub)
        dca.attention(cfg, q, qp, k, workspace=ws, out=out, lse=lse)
    end.record()
    dca.set_stage_events(None)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    stages = np.array([[ev.ms(6 * s + i, 6 * s + i + 1) for i in range(5)] for s in range(steps)])
    del ws, q, k
    return total_ms / steps, stages.mean(axis=0)


def cpu_baseline(w, inp, n_rows, seed=0):
    import oracle
    rng = np.random.default_rng(seed)
    T = w.T
    # rows spread uniformly over the sequence, so the mean key count matches the workload's
    ts = np.unique(((np.arange(n_rows) + rng.random(n_rows)) * T / n_rows).astype(np.int64))
    rows = ts  # B = 1 for prefill workloads; for decode rows are (b, 0)
    if w.T == 1:
        rows = np.arange(min(w.B, n_rows), dtype=np.int64)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    ff = inp["freq_factors"].astype(np.float64)
    t0 = time.perf_counter()
    oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=w.chunk, n_rot=w.n_rot, theta=w.theta,
                     scale=w.scale, freq_factors=ff, rows=rows, per_regime=False, n_threads=threads)
    dt = time.perf_counter() - t0
    return dict(value=len(rows) / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{len(rows)} of {w.B * w.T} query rows (all {w.Hq} heads), rows spread "
                       f"uniformly over the sequence; {dt:.1f} s on {threads} threads")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill-32k-c8192")
    ap.add_argument("--decode-workload", default="decode-b8-kv256k-c65536")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--cpu-rows", type=int, default=96)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for the traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (see DESIGN.md for how it "
              "would shard); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from dual_chunk_attention_amd import dca, synth

    w = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(w)
    ms, stages = time_leg(torch, dca, w, inp, args.steps, args.warmup)
    flops, _ = algorithmic_work(w)
    attn_ms = stages[3]
    achieved = flops / (attn_ms * 1e-3) / 1e12
    rec = {
        "metric": "DCA attn tokens/s: 32k prefill & 256k-KV decode; % MFMA / HBM peak",
        "value": w.B * w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K rounded to bf16; freq_factors U[1,8))",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "n_kv": w.N, "chunk": w.chunk,
                   "heads_q": w.Hq, "heads_kv": w.Hkv, "head_dim": w.D, "n_rot": w.n_rot},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("attn_prefill.hip") if w.name == "prefill-32k-c8192" else None,
                     "kernel": "attn_prefill_kernel (3 regime passes, one launch)",
                     "kernel_ms": attn_ms, "algorithmic_flop": flops},
        "stages_ms": {"remap": stages[0], "rope_q": stages[1], "rope_k": stages[2],
                      "regime_passes": stages[3], "merge": stages[4]},
    }
    del inp
    if not args.no_decode:
        wd = synth.WORKLOADS[args.decode_workload]
        inpd = synth.make_inputs(wd)
        msd, std = time_leg(torch, dca, wd, inpd, args.decode_steps, args.warmup)
        _, kv_bytes = algorithmic_work(wd)
        gbps = kv_bytes / (std[3] * 1e-3) / 1e9
        rec["decode"] = {
            "workload": wd.name, "value": wd.B * wd.T / (msd * 1e-3), "unit": "tokens/s",
            "ms_per_step": msd, "steps": args.decode_steps,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("attn_decode.hip") if wd.name == "decode-b8-kv256k-c65536" else None,
                         "kernel": "attn_decode_kernel (split-KV, 3 regimes)", "kernel_ms": std[3],
                         "algorithmic_bytes": kv_bytes},
            "stages_ms": {"remap": std[0], "rope_q": std[1], "tables": std[2],
                          "regime_passes": std[3], "merge": std[4]},
        }
        del inpd
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = int(src.numel() * 4)
        del src, dst
    if not args.no_cpu_baseline:
        inp = synth.make_inputs(w)
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_rows)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
