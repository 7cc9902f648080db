"""Benchmark of the Dual Chunk Attention hot path on one MI355X.

One step = one dca_attention call (remap, query rotation x3, key rotation, the three regime passes,
the N-way merge) on the 32k-token prefill workload (one global layer: 16 query heads, 2 KV heads,
head_dim 512, chunk 8192, bf16, inputs resident in HBM).  The 256k-KV decode workload (8 sequences,
chunk 65536) is timed as a second leg, the same decode over q8_0 and q4_0 key caches as third and
fourth legs, and with its cache split into a GPU window and a pinned-host tail as a fifth.  The 4k
prefill (chunk 1024) and the 1M-key prefill slice (4096 queries at positions [1044480, 1048576)
against 1048576 keys, chunk 65536) are timed as further prefill legs.  Prints one JSON line.

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
HOST_LINK_PEAK_GBPS = 64.0        # PCIe 5.0 x16, one direction


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


def measured_traffic(kernel_file, workload):
    """HBM bytes per launch of a kernel on a workload, from the FETCH_SIZE/WRITE_SIZE counter passes
    recorded in profiles/traffic.json (keyed "file:workload"); None when there is no record or the
    kernel source changed since the counters were taken."""
    key = f"{kernel_file}:{workload}"
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[key]
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
    the three regimes).  Decode: the cache read once (K = V): B*N*Hkv*D*2 bytes for bf16,
    B*N*Hkv*(D + 2*D/32) for q8_0 (one int8 code per dim, one fp16 scale per 32 dims) and
    B*N*Hkv*(D/2 + 2*D/32) for q4_0 (4-bit codes)."""
    i = w.q0 + np.arange(w.T, dtype=np.float64)
    pairs = float(np.minimum(i + 1, w.N).sum()) * w.B
    flops = 4.0 * w.D * w.Hq * pairs
    row_bytes = {"q8_0": w.D + 2 * (w.D // 32), "q4_0": w.D // 2 + 2 * (w.D // 32)}.get(w.dtype, w.D * 2)
    kv_bytes = float(w.B) * w.N * w.Hkv * row_bytes
    return flops, kv_bytes


def time_leg(torch, dca, w, inp, steps, warmup, n_win=None):
    """Time `steps` calls of the workload's entry point; n_win: bf16 cache split into cells
    [0, n_win) on the GPU and the rest in pinned host memory (dca_attention_window)."""
    cfg = dca.Config(head_dim=w.D, n_rot=w.n_rot, n_head_q=w.Hq, n_head_kv=w.Hkv, chunk=w.chunk,
                     rope_theta=w.theta, scale=w.scale, freq_factors=to_dev(torch, inp["freq_factors"]))
    q, qp = to_dev(torch, inp["q"]), to_dev(torch, inp["q_pos"])
    if n_win is not None:
        kb = torch.from_numpy(inp["k"].view(np.int16)).view(torch.bfloat16)
        k = (dca.Region(dca.KV_BF16, kb[:, :n_win].contiguous().to("cuda:0")),
             dca.Region(dca.KV_BF16, kb[:, n_win:].contiguous().pin_memory()))
        ws_bytes = dca.attention_window_workspace_size(cfg, w.B, w.T, n_win, w.N - n_win)
        call = dca.attention_window
    elif w.dtype in ("q8_0", "q4_0"):
        k = (to_dev(torch, inp["k_codes"]), to_dev(torch, inp["k_scales"].view(np.int16)))
        ws_bytes = dca.attention_q8_workspace_size(cfg, w.B, w.T, w.N)
        call = dca.attention_q8 if w.dtype == "q8_0" else dca.attention_q4
    else:
        k = (to_dev(torch, inp["k"]),)
        ws_bytes = dca.attention_workspace_size(cfg, q.dtype, w.B, w.T, w.N)
        call = dca.attention
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    out = torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.T, w.Hq), dtype=torch.float32, device="cuda:0")
    for _ in range(warmup):
        call(cfg, q, qp, *k, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    ev = HipEvents(6 * steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(steps):
        sub = (ctypes.c_void_p * 6)(*ev.arr[6 * s:6 * s + 6])
        dca.set_stage_events(sub)
        call(cfg, q, qp, *k, workspace=ws, out=out, lse=lse)
    end.record()
    dca.set_stage_events(None)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    stages = np.array([[ev.ms(6 * s + i, 6 * s + i + 1) for i in range(5)] for s in range(steps)])
    del ws, q, k
    return total_ms / steps, stages.mean(axis=0)


def sample_rows(w, n_rows, seed=0):
    """Query rows for the oracle timing: every chunk at local offsets {0, 1, c/2, c-2, c-1}, then
    uniformly drawn rows up to n_rows (prefill); all B rows (decode)."""
    if w.T == 1:
        return np.arange(w.B, dtype=np.int64)
    rng = np.random.default_rng(seed)
    pos = w.q0 + np.arange(w.T, dtype=np.int64)
    picked = set()
    for c0 in range(int(pos[0] // w.chunk) * w.chunk, int(pos[-1]) + 1, w.chunk):
        for off in (0, 1, w.chunk // 2, w.chunk - 2, w.chunk - 1):
            p = c0 + off
            if pos[0] <= p <= pos[-1]:
                picked.add(int(p - w.q0))
    rest = np.setdiff1d(np.arange(w.T), np.fromiter(picked, dtype=np.int64, count=len(picked)))
    extra = max(0, n_rows - len(picked))
    if extra:
        picked.update(int(t) for t in rng.choice(rest, size=min(extra, rest.size), replace=False))
    return np.array(sorted(picked), dtype=np.int64)


def cpu_baseline(w, inp, n_rows, seed=0):
    """The fp64 CPU oracle, timed on a sample of query rows of the same workload (all heads), on
    every host thread.  Reported as attended (query, key) pairs per second and as the query
    tokens per second that rate gives on the full workload."""
    import oracle
    rows = sample_rows(w, n_rows, seed)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    ff = inp["freq_factors"].astype(np.float64)
    t0 = time.perf_counter()
    oracle.attention(inp["q"], inp["q_pos"], inp["k"], chunk=w.chunk, n_rot=w.n_rot, theta=w.theta,
                     scale=w.scale, freq_factors=ff, rows=rows, per_regime=False, n_threads=threads)
    dt = time.perf_counter() - t0
    qpos = inp["q_pos"].reshape(-1).astype(np.float64)
    keys = np.minimum(qpos + 1, w.N)
    pairs_sample = float(keys[rows].sum()) * w.Hq
    pairs_full_per_token = float(keys.sum()) / keys.size * w.Hq
    pairs_per_s = pairs_sample / dt
    return dict(value=pairs_per_s / pairs_full_per_token, unit="tokens/s", cores=threads, kind="oracle",
                pairs_per_s=pairs_per_s,
                sample=f"{len(rows)} of {w.B * w.T} query rows x {w.Hq} heads ({pairs_sample:.3g} pairs): "
                       f"every chunk at local offsets 0, 1, c/2, c-2, c-1 plus uniform rows; {dt:.1f} s "
                       f"on {threads} threads (fp64 oracle incl. its key rotation); value = measured "
                       f"pairs/s over the workload's mean pairs per token")


def measured_peaks(torch, dca):
    """Reference rates measured on the device from the library's probe kernels (include/dca_calibrate.h): bf16
    MFMA 32x32x16 with no memory traffic (2048 workgroups of 4 waves), and a streaming read of
    4 GiB with 16-byte loads (8192 workgroups)."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3
    n_wg, iters = 2048, 2000
    sink = torch.empty((8192 * 256,), dtype=torch.float32, device="cuda:0")
    t = timed(lambda: dca.probe_mfma_bf16(n_wg, iters, sink), 5)
    mfma = n_wg * 4 * iters * 32 * 32768.0 / t / 1e12
    x = torch.empty((1 << 32,), dtype=torch.uint8, device="cuda:0")
    x.fill_(1)
    t = timed(lambda: dca.probe_hbm_read(x, 8192, sink), 10)
    read = x.numel() / t / 1e9
    del x
    # host link: a 1 GiB copy from pinned host memory, and the same streaming-read kernel reading
    # pinned host memory in place
    h = torch.ones((1 << 30,), dtype=torch.uint8).pin_memory()
    dst = torch.empty((1 << 30,), dtype=torch.uint8, device="cuda:0")
    t = timed(lambda: dst.copy_(h, non_blocking=True), 5)
    h2d = h.numel() / t / 1e9
    t = timed(lambda: dca.probe_hbm_read(h, 8192, sink), 3)
    host_read = h.numel() / t / 1e9
    del h, dst, sink
    return {"mfma_bf16_tflops": mfma, "hbm_read_gbps": read, "host_copy_gbps": h2d,
            "host_read_gbps": host_read,
            "how": "dca_probe_mfma_bf16 (2048 x 4 waves, 32x32x16 bf16, no memory traffic); "
                   "dca_probe_hbm_read over 4 GiB; 1 GiB pinned host -> device copy; "
                   "dca_probe_hbm_read over 1 GiB of pinned host memory"}


def prefill_leg(torch, dca, synth, name, steps, warmup, cpu_rows):
    """One prefill workload: tokens/s of whole dca_attention calls, the fused pass's roofline, and
    (cpu_rows > 0) the oracle timed on a sample of its rows."""
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    ms, st = time_leg(torch, dca, w, inp, steps, warmup)
    flops, _ = algorithmic_work(w)
    achieved = flops / (st[3] * 1e-3) / 1e12
    leg = {
        "workload": w.name, "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
        "steps": steps,
        "config": {"workload": w.name, "B": w.B, "T": w.T, "q0": w.q0, "n_kv": w.N, "chunk": w.chunk,
                   "heads_q": w.Hq, "heads_kv": w.Hkv, "head_dim": w.D, "n_rot": w.n_rot},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("attn_fused.hip", w.name),
                     "kernel": "attn_fused_kernel (the three regimes in one pass, one launch)",
                     "kernel_ms": st[3], "algorithmic_flop": flops},
        "stages_ms": {"remap": st[0], "rope_q": st[1], "rope_k": st[2], "regime_passes": st[3],
                      "merge": st[4]},
    }
    if cpu_rows > 0:
        leg["cpu_baseline"] = cpu_baseline(w, inp, cpu_rows)
    del inp
    return leg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill-32k-c8192")
    ap.add_argument("--decode-workload", default="decode-b8-kv256k-c65536")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--q8-workload", default="decode-b8-kv256k-c65536-q8")
    ap.add_argument("--q4-workload", default="decode-b8-kv256k-c65536-q4")
    ap.add_argument("--no-q8", action="store_true")
    ap.add_argument("--no-q4", action="store_true")
    ap.add_argument("--window-cells", type=int, default=65536,
                    help="window leg: cells of the 256k decode cache kept on the GPU (the rest in pinned host memory)")
    ap.add_argument("--window-steps", type=int, default=5)
    ap.add_argument("--no-window", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=768)
    ap.add_argument("--extra-prefill", default="prefill-4k-c1024:512,prefill-4k-at-1m-c65536:4",
                    help="further prefill legs as workload:cpu_rows, comma-separated ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-measured-peaks", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for the traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (a layer would shard by KV "
              "head, one or more of the 2 per GPU, or split the key cache across GPUs and merge the "
              "partials by their LSE); run with --gpus 1.", file=sys.stderr)
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
                     "traffic": measured_traffic("attn_fused.hip", w.name),
                     "kernel": "attn_fused_kernel (the three regimes in one pass, one launch)",
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
                         "traffic": measured_traffic("attn_decode.hip", wd.name),
                         "kernel": "attn_decode_kernel (split-KV, 3 regimes)", "kernel_ms": std[3],
                         "algorithmic_bytes": kv_bytes},
            "stages_ms": {"remap": std[0], "rope_q": std[1], "tables": std[2],
                          "regime_passes": std[3], "merge": std[4]},
        }
        if not args.no_window:
            nw = args.window_cells
            msw, stw = time_leg(torch, dca, wd, inpd, args.window_steps, 1, n_win=nw)
            host_bytes = float(wd.B) * (wd.N - nw) * wd.Hkv * wd.D * 2
            gbw = host_bytes / (stw[3] * 1e-3) / 1e9
            rec["decode_window"] = {
                "workload": f"{wd.name}, cells [0, {nw}) on the GPU, [{nw}, {wd.N}) in pinned host memory",
                "value": wd.B * wd.T / (msw * 1e-3), "unit": "tokens/s", "ms_per_step": msw,
                "steps": args.window_steps,
                "roofline": {"bound": "host_link", "achieved": gbw, "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                             "frac": gbw / HOST_LINK_PEAK_GBPS, "traffic": None,
                             "kernel": "attn_decode_kernel over the host tail, then over the window",
                             "kernel_ms": stw[3], "host_bytes": host_bytes,
                             "note": "achieved = tail bytes read over the host link / both region passes"},
                "stages_ms": {"remap": stw[0], "rope_q": stw[1], "tables": stw[2],
                              "regime_passes": stw[3], "merge": stw[4]},
            }
        del inpd
    for fmt, name in (("q8", args.q8_workload), ("q4", args.q4_workload)):
        if getattr(args, "no_" + fmt):
            continue
        wq = synth.WORKLOADS[name]
        inpq = synth.make_inputs(wq)
        msq, stq = time_leg(torch, dca, wq, inpq, args.decode_steps, args.warmup)
        _, q_bytes = algorithmic_work(wq)
        gbps = q_bytes / (stq[3] * 1e-3) / 1e9
        rec["decode_" + fmt] = {
            "workload": wq.name, "value": wq.B * wq.T / (msq * 1e-3), "unit": "tokens/s",
            "ms_per_step": msq, "steps": args.decode_steps,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("attn_decode_quant.hip", wq.name),
                         "kernel": f"attn_decode_quant_kernel<{8 if fmt == 'q8' else 4}> (split-KV over the "
                                   f"{wq.dtype} cache, 3 regimes)",
                         "kernel_ms": stq[3], "algorithmic_bytes": q_bytes},
            "stages_ms": {"remap": stq[0], "rope_q": stq[1], "tables": stq[2],
                          "regime_passes": stq[3], "merge": stq[4]},
        }
        del inpq
    for spec in [x for x in args.extra_prefill.split(",") if x]:
        name, _, n_cpu = spec.partition(":")
        leg = prefill_leg(torch, dca, synth, name, args.steps, args.warmup,
                          0 if args.no_cpu_baseline else int(n_cpu or 0))
        rec["prefill_" + name.split("-c")[0].replace("prefill-", "").replace("-", "_")] = leg
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = int(src.numel() * 4)
        del src, dst
    if not args.no_measured_peaks:
        pk = measured_peaks(torch, dca)
        rec["roofline"]["measured_peak"] = pk["mfma_bf16_tflops"]
        rec["roofline"]["frac_of_measured_peak"] = rec["roofline"]["achieved"] / pk["mfma_bf16_tflops"]
        if "decode" in rec:
            rd = rec["decode"]["roofline"]
            rd["measured_peak"] = pk["hbm_read_gbps"]
            rd["frac_of_measured_peak"] = rd["achieved"] / pk["hbm_read_gbps"]
        for key in ("decode_q8", "decode_q4"):
            if key in rec:
                rq = rec[key]["roofline"]
                rq["measured_peak"] = pk["hbm_read_gbps"]
                rq["frac_of_measured_peak"] = rq["achieved"] / pk["hbm_read_gbps"]
        for key in [k for k in rec if k.startswith("prefill_")]:
            rp = rec[key]["roofline"]
            rp["measured_peak"] = pk["mfma_bf16_tflops"]
            rp["frac_of_measured_peak"] = rp["achieved"] / pk["mfma_bf16_tflops"]
        if "decode_window" in rec:
            rw = rec["decode_window"]["roofline"]
            rw["measured_peak"] = pk["host_read_gbps"]
            rw["frac_of_measured_peak"] = rw["achieved"] / pk["host_read_gbps"]
        rec["measured_peaks"] = pk
    if not args.no_cpu_baseline:
        inp = synth.make_inputs(w)
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_rows)
        del inp
        if "decode" in rec:
            inpd = synth.make_inputs(synth.WORKLOADS[args.decode_workload])
            rec["decode"]["cpu_baseline"] = cpu_baseline(synth.WORKLOADS[args.decode_workload], inpd, args.cpu_rows)
            del inpd
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
