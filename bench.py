"""Benchmark of the whole hot path on one MI355X.

A step is one pass of every stage over the batch workload (Qwen3-0.6B-shaped, 32
sequences with ragged cached lengths drawn uniformly from [128, 8192]):
  1. kv_append_rope  RoPE + in-place append of a 4,096-token continuation on sequence 0
  2. gqa_attn_prefill causal attention of those 4,096 tokens (fp32 MFMA)
  3. a 512 MB streaming read (cache flush: the decode below then reads its window from
     HBM, not from the 256 MB Infinity Cache the prefill has just filled)
  4. kv_append_rope  RoPE + append of one token for each of the 32 sequences
  5. gqa_attn_decode split-K decode attention for the 32 sequences (+ combine)
Inputs are resident in HBM before the timed region; the timed region is K steps,
bracketed by device synchronisation.  HIP events on the library's stream time each
stage.

Reported:
  value          decode attention KV GB/s, cold: algorithmic K+V bytes of the 32 windows
                 (sum_b (pos_b + 1) * 2 * n_head_kv * hd_kv * bytes per value: 4 for f32,
                 2 for binary16, 34/32 for Q8_0) / decode-attention time (stage 5)
  prefill_tflops algorithmic prefill FLOPs (4 * n_head * hd_kv * sum_t (pos_t + 1)) /
                 prefill-attention time
  roofline       the dominant kernel (prefill, MFMA-bound) against the fp32 matrix peak;
  roofline_decode the decode kernels against HBM bandwidth and against the measured
                 streaming-read ceiling; `traffic` in both is HBM bytes per launch from
                 copy-calibrated FETCH_SIZE + WRITE_SIZE counters recorded in profiles/
                 (null once the kernel sources differ from the profiled ones)
  read_ceiling   a plain streaming read of 1 GiB (ordinary and nontemporal loads)
  long_context   the Qwen3-0.6B long-context decode (32,767 cached rows, one layer),
                 cold, at the API (HIP events) and per kernel (split, merge) from a
                 torch.profiler pass (kernel durations of the step's kernels are in the
                 rocprofv3 summaries under profiles/: under torch.profiler the MFMA-bound
                 prefill ran ~13% slower than under events or rocprofv3, the memory-bound
                 decode kernels did not)
  cpu_baseline   the plain C oracle on the host cores, on bounded samples

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 15] [--no-cpu-baseline]
                       [--no-long-context] [--kv f32|f16|q8_0] [--decode-runs] [--fused-qkv]
       python bench.py --workload long|layer|stack [--graph]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn KV GB/s (% HBM peak) and prefill attn TFLOP/s, Qwen3-0.6B shape"
HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
FLUSH_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class ReadProbe:
    """The streaming-read helper (lib/libkvc_probe.so): the read ceiling, and the cache
    flush between timed calls (a read, so no dirty lines are left behind)."""

    def __init__(self, dev):
        import torch
        path = os.path.join(ROOT, "kv_cache_causal_amd", "lib", "libkvc_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build()")
        self.L = ctypes.CDLL(path)
        self.L.kvc_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_void_p]
        self.L.kvc_probe_stream_read.restype = ctypes.c_int
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        self.sink = torch.zeros(8192, dtype=torch.float32, device=dev)

    def read(self, nbytes, nontemporal=False, blocks=2048, unroll=1, src=None):
        import kv_cache_causal_amd as kvc
        src = self.buf if src is None else src
        e = self.L.kvc_probe_stream_read(src.data_ptr(), int(nbytes), self.sink.data_ptr(),
                                         blocks, int(nontemporal), unroll, kvc._stream(None))
        if e != 0:
            raise RuntimeError(f"stream read probe failed: hipError {e}")

    def flush(self):
        self.read(FLUSH_BYTES)

    def ceiling(self, reps=10):
        """Median GB/s of cold 1 GiB streaming reads (each after a 512 MB read of another
        buffer): the best of 1 or 2 loads per trip and 1024 / 2048 / 4096 workgroups, per
        load kind."""
        import torch
        other = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=self.buf.device)
        res = {}
        for nt in (False, True):
            best, shape = 0.0, None
            for unroll in (1, 2):
                for blocks in (1024, 2048, 4096):
                    evs = [(torch.cuda.Event(enable_timing=True),
                            torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
                    for a, b in evs:
                        self.read(FLUSH_BYTES, src=other)
                        a.record()
                        self.read(self.buf.numel() * 4, nt, blocks, unroll)
                        b.record()
                    torch.cuda.synchronize()
                    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
                    gbs = self.buf.numel() * 4 / (ms * 1e-3) / 1e9
                    if gbs > best:
                        best, shape = gbs, f"{unroll} load(s) per trip, {blocks} workgroups"
            key = "nontemporal" if nt else "plain"
            res[key + "_gbs"] = round(best, 1)
            res[key + "_shape"] = shape
        del other
        return res


def kernel_averages(fn, reps):
    """Run fn() `reps` times under torch.profiler; per kernel name (template arguments
    kept, namespaces and parameter list dropped): median and mean device time (us) and
    launches per rep."""
    import torch
    from torch.profiler import ProfilerActivity, profile
    fn()
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
    times = {}
    for e in prof.events():
        if e.device_type.name != "CUDA" or "kvc::" not in e.name:
            continue
        name = e.name.replace("(anonymous namespace)", "").split("(")[0].split("::")[-1]
        t = getattr(e, "device_time", None)
        times.setdefault(name, []).append(e.cuda_time if t is None else t)
    return {n: {"median_us": round(float(np.median(t)), 2), "mean_us": round(float(np.mean(t)), 2),
                "launches_per_rep": len(t) // reps} for n, t in sorted(times.items())}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The GPU's clock ramps up over the first ~25 ms of sustained work: in a kernel trace of
    # this step the prefill kernel took 2.16 ms on its first launch and settled at
    # 1.83-1.85 ms from about the twelfth.  Fifteen untimed steps (~35 ms) reach that state.
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the long-context decode object of the default run")
    ap.add_argument("--no-kernel-trace", action="store_true",
                    help="skip the torch.profiler pass that splits the long-context decode "
                         "into its split and merge kernels")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="target wall time of the oracle's decode sample")
    ap.add_argument("--kv", choices=["f32", "f16", "q8_0"], default="f32",
                    help="region format: f32, binary16 (half the bytes) or Q8_0 (34 bytes per 32 "
                         "values); the arithmetic is f32 in every case")
    ap.add_argument("--decode-runs", action="store_true",
                    help="stage 5 through gqa_attn_decode_runs: each sequence's window given "
                         "as two explicit runs, its second half first")
    ap.add_argument("--fused-qkv", action="store_true",
                    help="stage 4 through kv_qkv_rope_append: the 32 decode tokens' q/k/v are "
                         "projected from d_model=1024 inputs with synthetic weights, rotated "
                         "and stored in one kernel")
    ap.add_argument("--workload", choices=["batch", "long", "layer", "stack"], default="batch",
                    help="batch: the 32-sequence Qwen3-0.6B step (default, the headline); "
                         "long: one decode over 32,767 cached rows; layer: one Qwen2.5-0.5B "
                         "layer decode at 511; stack: 28-layer Qwen3-0.6B prefill of 511 and "
                         "decode steps (f32 regions; cold = 512 MB read between steps)")
    ap.add_argument("--graph", action="store_true",
                    help="with --workload long|layer|stack: replay each step's appends and "
                         "decodes from HIP graphs captured once, so the host's per-call "
                         "launch time is not measured")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB device-to-device copy before timing, so that "
                         "HBM counters (FETCH_SIZE / WRITE_SIZE) can be calibrated against "
                         "a kernel of known traffic in the same profiler run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_causal_amd as kvc
    from tests import workloads as W

    if args.workload != "batch":
        other_workload(args)
        return

    w = W.QWEN3_BATCH
    nt = w.extra["prefill"]
    n_past = W.batch_n_past(w)
    pre_pos = np.arange(n_past[0], n_past[0] + nt, dtype=np.int32)
    lens = n_past.copy()
    lens[0] += nt
    seqs = np.arange(w.n_seq, dtype=np.int32)
    # Bytes per cached value: f32 4, binary16 2, Q8_0 34/32 (a code plus its share of the
    # block's 2-byte scale).
    esize = {"f32": 4, "f16": 2, "q8_0": 34 / 32}[args.kv]
    kv_bytes = int(int((lens.astype(np.int64) + 1).sum()) * 2 * w.n_head_kv * w.hd_kv * esize)
    pre_flops = 4 * w.n_head * w.hd_kv * int((pre_pos.astype(np.int64) + 1).sum())

    torch.cuda.init()
    kvc.lib()
    dev = torch.device("cuda:0")
    probe = ReadProbe(dev)
    log(f"bench: workload {w.name}; filling {int(n_past.sum())} cached rows")
    t0 = time.time()
    kv_dtype = {"f32": kvc.KV_F32, "f16": kvc.KV_F16, "q8_0": kvc.KV_Q8_0}[args.kv]
    cache = kvc.kv_alloc(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity, dtype=kv_dtype)
    orc_cache = None
    if not args.no_cpu_baseline:
        from oracle import OracleCache
        orc_cache = OracleCache(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity,
                                dtype=kv_dtype)
    chunk = w.extra["fill_chunk"]
    for s in range(w.n_seq):
        for ci, r0 in enumerate(range(0, int(n_past[s]), chunk)):
            r1 = min(int(n_past[s]), r0 + chunk)
            k, v = W.fill_rows(w, s, 0, ci, r1 - r0)
            k = k.reshape(r1 - r0, w.n_head_kv, w.hd_kv)
            v = v.reshape(r1 - r0, w.n_head_kv, w.hd_kv)
            rows = np.arange(r0, r1, dtype=np.int32)
            kvc.kv_append_rope(cache, 0, np.full(r1 - r0, s, np.int32), rows, None, 0, 0,
                               torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                               w.base, w.freq_scale, w.style)
            if orc_cache is not None:
                orc_cache.append_rope(0, np.full(r1 - r0, s, np.int32), rows, None, 0, 0, k, v,
                                      w.base, w.freq_scale, w.style)
    qp, kp, vp = (torch.from_numpy(a).to(dev) for a in W.prefill_qkv(w, nt, 0, 0))
    qd, kd, vd = (torch.from_numpy(a).to(dev) for a in W.decode_qkv(w, w.n_seq, 0, 0))
    out_pre = torch.empty((nt, w.n_head, w.hd_kv), dtype=torch.float32, device=dev)
    out_dec = torch.empty((w.n_seq, w.n_head, w.hd_kv), dtype=torch.float32, device=dev)
    # Fused-step inputs: Qwen3-0.6B's hidden width, seeded N(0, 1/d) weights (synthetic).
    D_MODEL = 1024
    qkv_rows = (w.n_head * w.hd, w.n_head_kv * w.hd_kv, w.n_head_kv * w.hd_kv)
    if args.fused_qkv:
        wts = [torch.from_numpy(W.custom(900 + i, (r, D_MODEL)) * np.float32(D_MODEL ** -0.5)).to(dev)
               for i, r in enumerate(qkv_rows)]
        x_dec = torch.from_numpy(W.custom(910, (w.n_seq, D_MODEL))).to(dev)
    torch.cuda.synchronize()
    log(f"bench: setup {time.time() - t0:.1f}s; n_past[0] {n_past[0]}, "
        f"prefill {pre_flops / 1e9:.1f} GFLOP, decode {kv_bytes / 1e9:.3f} GB KV")

    ceiling = probe.ceiling()
    log(f"bench: streaming-read ceiling {ceiling}")

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: copy probe: 1 GiB read + 1 GiB written by one copy kernel")
        del src, dst

    nsteps = args.warmup + args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(nsteps)]

    # The same windows as explicit runs: [L/2, L) then [0, L/2) for window length L.
    win_runs = [[(int(x + 1) // 2, int(x + 1) - int(x + 1) // 2), (0, int(x + 1) // 2)]
                for x in lens]

    def decode():
        if args.decode_runs:
            kvc.gqa_attn_decode_runs(cache, 0, seqs, win_runs, qd, w.n_head, w.hd, w.scale,
                                     out_dec)
        else:
            kvc.gqa_attn_decode(cache, 0, seqs, lens, qd, w.n_head, w.hd, w.scale, out_dec)

    def step(e=None):
        rec = (lambda i: e[i].record()) if e is not None else (lambda i: None)
        rec(0)
        kvc.kv_append_rope(cache, 0, np.zeros(nt, np.int32), pre_pos, qp, w.n_head, w.hd, kp, vp,
                           w.base, w.freq_scale, w.style)
        rec(1)
        kvc.gqa_attn_prefill(cache, 0, 0, pre_pos, qp, w.n_head, w.hd, w.scale, out_pre)
        rec(2)
        probe.flush()
        rec(3)
        if args.fused_qkv:
            kvc.kv_qkv_rope_append(cache, 0, seqs, lens, x_dec, wts[0], None, wts[1], None,
                                   wts[2], None, w.n_head, w.hd, qd, w.base, w.freq_scale,
                                   w.style)
        else:
            kvc.kv_append_rope(cache, 0, seqs, lens, qd, w.n_head, w.hd, kd, vd, w.base,
                               w.freq_scale, w.style)
        rec(4)
        decode()
        rec(5)

    for i in range(args.warmup):
        step(ev[i])
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done; timing {args.steps}")
    t_start = time.perf_counter()
    for i in range(args.warmup, nsteps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    timed = ev[args.warmup:]
    ms = lambda a, b: np.array([e[a].elapsed_time(e[b]) for e in timed])  # noqa: E731
    t_app_pre, t_pre, t_flush, t_app_dec, t_dec = ms(0, 1), ms(1, 2), ms(2, 3), ms(3, 4), ms(4, 5)
    t_step = ms(0, 5)
    ms_per_step = wall * 1e3 / args.steps
    dec_gbs = kv_bytes / (t_dec.mean() * 1e-3) / 1e9
    pre_tflops = pre_flops / (t_pre.mean() * 1e-3) / 1e12
    app_bytes = nt * (2 * w.n_head * w.hd + 2 * w.n_head_kv * w.hd_kv) * 4 + \
        nt * 2 * w.n_head_kv * w.hd_kv * esize
    log(f"bench: step {ms_per_step:.3f} ms (events {t_step.mean():.3f}); append+rope(4096) "
        f"{t_app_pre.mean() * 1e3:.1f} us, prefill {t_pre.mean():.3f} ms, flush "
        f"{t_flush.mean() * 1e3:.1f} us, append(32) {t_app_dec.mean() * 1e3:.1f} us, decode "
        f"(cold) {t_dec.mean() * 1e3:.1f} us")

    # Warm decode for context: the same call back to back (the 1.1 GB of windows exceed the
    # 256 MB Infinity Cache, so little of it can stay resident).
    warm_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for a, b in warm_ev:
        a.record()
        decode()
        b.record()
    torch.cuda.synchronize()
    t_dec_warm = np.array([a.elapsed_time(b) for a, b in warm_ev])

    result = {
        "metric": METRIC,
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # arithmetic; the region format is config.kv_dtype
        "data": "synthetic (seeded N(0,1) q/k/v and cache rows)",
        "config": {
            "workload": "qwen3-0.6b-batch: 32 sequences, 16 q heads / 8 kv heads, head dim 128, "
                        "ragged n_past U[128,8192]; 4096-token continuation prefill on seq 0 + "
                        "one decode step for all 32 (512 MB read between them: cold decode)",
            "kv_dtype": args.kv,
            "decode_windows": "explicit runs, 2 per sequence" if args.decode_runs else
                              "position-derived [0, pos]",
            "decode_append": "fused projections + RoPE + store" if args.fused_qkv else
                             "kv_append_rope of given q/k/v",
            "n_seq": int(w.n_seq), "n_head": w.n_head, "n_head_kv": w.n_head_kv,
            "hd": w.hd, "hd_kv": w.hd_kv, "capacity": w.capacity,
            "n_past_seq0": int(n_past[0]), "prefill_tokens": nt,
            "decode_window_rows": int((lens.astype(np.int64) + 1).sum()),
        },
        "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_hbm_frac_cold": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_gbs_warm": round(kv_bytes / (t_dec_warm.mean() * 1e-3) / 1e9, 1),
        "prefill_tflops": round(pre_tflops, 3),
        "prefill_mfma_frac": round(pre_tflops / FP32_MFMA_PEAK_TFLOPS, 4),
        "stage_us": {
            "append_rope_4096": round(float(t_app_pre.mean()) * 1e3, 2),
            "prefill_attn": round(float(t_pre.mean()) * 1e3, 2),
            "flush_read_512MB": round(float(t_flush.mean()) * 1e3, 2),
            "append_rope_32": round(float(t_app_dec.mean()) * 1e3, 2),
            "decode_attn": round(float(t_dec.mean()) * 1e3, 2),
            "decode_attn_median": round(float(np.median(t_dec)) * 1e3, 2),
            "decode_attn_warm": round(float(t_dec_warm.mean()) * 1e3, 2),
        },
        "append_gbs": round(app_bytes / (t_app_pre.mean() * 1e-3) / 1e9, 1),
        "read_ceiling": {**ceiling, "what": "cold 1 GiB grid-stride float4 read "
                                            "(lib/libkvc_probe.so), best launch shape, median "
                                            "of 10"},
        **({"fused_qkv": {
            "what": "kv_qkv_rope_append of the 32 decode tokens, d_model 1024, no biases",
            "us": round(float(t_app_dec.mean()) * 1e3, 2),
            "weight_bytes": 4 * D_MODEL * sum(qkv_rows),
            "weight_gbs": round(4 * D_MODEL * sum(qkv_rows) / (t_app_dec.mean() * 1e-3) / 1e9, 1),
        }} if args.fused_qkv else {}),
        "roofline": {
            "kernel": "prefill_kernel<128> (gqa_attn_prefill)",
            "bound": "mfma",
            "achieved": round(pre_tflops, 3),
            "peak": FP32_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_tflops / FP32_MFMA_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("prefill") if args.kv == "f32" else None,
            "flops_per_launch": pre_flops,
            "avg_launch_us": round(float(t_pre.mean()) * 1e3, 2),
        },
        "roofline_decode": {
            "kernel": "decode_split_kernel<128,2> + decode_combine_kernel<128> (" +
                      ("gqa_attn_decode_runs)" if args.decode_runs else "gqa_attn_decode)") +
                      ", cold",
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "frac_of_read_ceiling": round(dec_gbs / ceiling["nontemporal_gbs"], 4),
            "traffic": measured_traffic("decode") if args.kv == "f32" and not args.decode_runs
            else None,
            "bytes_per_launch": kv_bytes,
            "avg_launch_us": round(float(t_dec.mean()) * 1e3, 2),
        },
    }
    if not args.no_long_context:
        result["long_context"] = long_context(probe, args.steps, not args.no_kernel_trace)
    if orc_cache is not None:
        result["cpu_baseline"] = cpu_baseline(orc_cache, w, seqs, lens, kv_bytes, pre_pos,
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


def long_context(probe, reps, trace):
    """The Qwen3-0.6B long-context decode: one layer, rows 0..32,766 cached, the token at
    32,767 appended, then decode over all 32,768 rows (268 MB of K and V), each timed call
    preceded by the 512 MB flush read (cold)."""
    import torch

    import kv_cache_causal_amd as kvc
    from tests import workloads as W
    w = W.QWEN3_LONG
    dev = torch.device("cuda:0")
    n_past = w.extra["n_past"]
    cache = kvc.kv_alloc(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity)
    chunk = w.extra["fill_chunk"]
    for ci, r0 in enumerate(range(0, n_past, chunk)):
        r1 = min(n_past, r0 + chunk)
        k, v = W.fill_rows(w, 0, 0, ci, r1 - r0)
        kvc.kv_append_rope(cache, 0, np.zeros(r1 - r0, np.int32), np.arange(r0, r1, dtype=np.int32),
                           None, 0, 0,
                           torch.from_numpy(k.reshape(r1 - r0, w.n_head_kv, w.hd_kv)).to(dev),
                           torch.from_numpy(v.reshape(r1 - r0, w.n_head_kv, w.hd_kv)).to(dev),
                           w.base, w.freq_scale, w.style)
    q, k, v = (torch.from_numpy(a).to(dev) for a in W.decode_qkv(w, 1, 0, 0))
    kvc.kv_append_rope(cache, 0, [0], [n_past], q, w.n_head, w.hd, k, v, w.base, w.freq_scale,
                       w.style)
    out = torch.empty((1, w.n_head, w.hd_kv), dtype=torch.float32, device=dev)
    win_bytes = (n_past + 1) * 2 * w.n_head_kv * w.hd_kv * 4

    def dec():
        kvc.gqa_attn_decode(cache, 0, [0], [n_past], q, w.n_head, w.hd, w.scale, out)

    for _ in range(3):
        probe.flush()
        dec()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        probe.flush()
        a.record()
        dec()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    res = {
        "workload": f"{w.name}: 1 layer, {w.n_head} q heads / {w.n_head_kv} kv heads, head dim "
                    f"{w.hd_kv}, decode at {n_past} over {n_past + 1} rows (capacity {w.capacity}), "
                    "512 MB read before each call",
        "bytes_per_call": win_bytes,
        "api_us_cold": round(float(t.mean()), 2),
        "api_us_cold_median": round(float(np.median(t)), 2),
        "gbs_cold": round(float(win_bytes / (t.mean() * 1e-6) / 1e9), 1),
        "hbm_frac_cold": round(float(win_bytes / (t.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS), 4),
    }
    if trace:
        def cold():
            probe.flush()
            dec()
        ks = kernel_averages(cold, 10)
        split = sum(v["median_us"] * v["launches_per_rep"] for n, v in ks.items()
                    if n.startswith("decode_split_kernel"))
        merge = sum(v["median_us"] * v["launches_per_rep"] for n, v in ks.items()
                    if n.startswith("decode_combine_kernel"))
        res["split_us"] = round(split, 2)
        res["merge_us"] = round(merge, 2)
        if split + merge > 0:
            res["kernels_gbs"] = round(win_bytes / ((split + merge) * 1e-6) / 1e9, 1)
            res["kernels_hbm_frac"] = round(res["kernels_gbs"] / HBM_PEAK_GBS, 4)
    log(f"bench: long context {res}")
    del cache
    return res


def other_workload(args):
    """The long-context, single-layer and 28-layer workloads: each step appends one token
    per layer, then decodes each layer; `cold` steps read 512 MB between steps (outside the
    timed events) so the cache is read from HBM.  The stack workload also times its
    28-layer prefill of 511 tokens once.  With --graph the appends and the decodes are
    each captured once into a HIP graph and replayed, which takes the host's per-call
    launch time out of the measurement."""
    import torch

    import kv_cache_causal_amd as kvc
    from tests import workloads as W

    w = {"long": W.QWEN3_LONG, "layer": W.QWEN25_LAYER, "stack": W.QWEN3_STACK}[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.init()
    kvc.lib()
    probe = ReadProbe(dev)
    cache = kvc.kv_alloc(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity)
    n_past = w.extra.get("n_past", w.extra.get("prefill"))
    log(f"bench: workload {w.name}; filling {n_past} rows x {w.n_layer} layers")
    pre_ev = None
    if args.workload == "stack":
        # The prefill itself is part of this workload: append + prefill of 511 per layer.
        pos = np.arange(n_past, dtype=np.int32)
        outp = torch.empty((n_past, w.n_head, w.hd_kv), dtype=torch.float32, device=dev)
        qkv = [[torch.from_numpy(a).to(dev) for a in W.prefill_qkv(w, n_past, layer)]
               for layer in range(w.n_layer)]
        pre_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for rep_ in range(2):   # the second pass is the timed one (tables built)
            qs = [t[0].clone() for t in qkv]   # the append rotates q in place
            torch.cuda.synchronize()
            pre_ev[0].record()
            for layer in range(w.n_layer):
                _, k, v = qkv[layer]
                kvc.kv_append_rope(cache, layer, np.zeros(n_past, np.int32), pos, qs[layer],
                                   w.n_head, w.hd, k, v, w.base, w.freq_scale, w.style)
                kvc.gqa_attn_prefill(cache, 0, layer, pos, qs[layer], w.n_head, w.hd, w.scale,
                                     outp)
            pre_ev[1].record()
        torch.cuda.synchronize()
    else:
        chunk = w.extra.get("fill_chunk", 4096)
        for ci, r0 in enumerate(range(0, n_past, chunk)):
            r1 = min(n_past, r0 + chunk)
            k, v = W.fill_rows(w, 0, 0, ci, r1 - r0)
            kvc.kv_append_rope(cache, 0, np.zeros(r1 - r0, np.int32),
                               np.arange(r0, r1, dtype=np.int32), None, 0, 0,
                               torch.from_numpy(k.reshape(r1 - r0, w.n_head_kv, w.hd_kv)).to(dev),
                               torch.from_numpy(v.reshape(r1 - r0, w.n_head_kv, w.hd_kv)).to(dev),
                               w.base, w.freq_scale, w.style)
    steps = [W.decode_qkv(w, 1, st % max(1, w.extra.get("decode_steps", 1)), layer)
             for st in range(1) for layer in range(w.n_layer)]
    dq = [[torch.from_numpy(a).to(dev) for a in t] for t in steps]
    out = torch.empty((1, w.n_head, w.hd_kv), dtype=torch.float32, device=dev)
    pos = np.array([n_past], np.int32)
    zero = np.zeros(1, np.int32)
    win_bytes = (n_past + 1) * 2 * w.n_head_kv * w.hd_kv * 4 * w.n_layer

    def appends():
        for layer in range(w.n_layer):
            q, k, v = dq[layer]
            kvc.kv_append_rope(cache, layer, zero, pos, q, w.n_head, w.hd, k, v, w.base,
                               w.freq_scale, w.style)

    def decodes():
        for layer in range(w.n_layer):
            kvc.gqa_attn_decode(cache, layer, zero, pos, dq[layer][0], w.n_head, w.hd, w.scale,
                                out)

    app, dec = appends, decodes
    if args.graph:
        # Warm up eagerly (tables, scratch sizes), then capture each half of the step once;
        # every replay launches the same kernels with the same arguments.
        for _ in range(2):
            appends()
            decodes()
        torch.cuda.synchronize()
        g_app, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_app):
            appends()
        with torch.cuda.graph(g_dec):
            decodes()
        torch.cuda.synchronize()
        app, dec = g_app.replay, g_dec.replay

    res = {}
    for mode in ("warm", "cold"):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.warmup + args.steps)]
        for ev in evs:
            if mode == "cold":
                # 512 MB read (not written: dirty lines would make the timed step pay for
                # their write-back) evicts the cache rows from L2 and the MALL.
                probe.flush()
            ev[0].record()
            app()
            ev[1].record()
            dec()
            ev[2].record()
        torch.cuda.synchronize()
        timed = evs[args.warmup:]
        step_us = np.array([e[0].elapsed_time(e[2]) * 1e3 for e in timed])
        dec_us = np.array([e[1].elapsed_time(e[2]) * 1e3 for e in timed])
        res[mode] = (float(step_us.mean()), float(dec_us.mean()))
        log(f"bench: {mode}: step {res[mode][0]:.1f} us, decode attention {res[mode][1]:.1f} us "
            f"over {w.n_layer} layer(s)" + (" (HIP graph replay)" if args.graph else ""))
    dec_gbs = win_bytes / (res["cold"][1] * 1e-6) / 1e9
    result = {
        "metric": METRIC, "value": round(dec_gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["cold"][0] / 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1) q/k/v and cache rows)",
        "config": {"workload": f"{w.name}: {w.n_layer} layer(s), {w.n_head} q heads / "
                               f"{w.n_head_kv} kv heads, head dim {w.hd_kv}, decode at {n_past} "
                               f"(cold: 512 MB read between steps)"
                               + ("; steps replayed from HIP graphs" if args.graph else ""),
                   "n_layer": w.n_layer, "n_past": n_past, "capacity": w.capacity},
        "decode_attn_us": {"cold": round(res["cold"][1], 2), "warm": round(res["warm"][1], 2)},
        "step_us": {"cold": round(res["cold"][0], 2), "warm": round(res["warm"][0], 2)},
        "decode_hbm_frac_cold": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_gbs_warm": round(win_bytes / (res["warm"][1] * 1e-6) / 1e9, 1),
        "roofline": {"kernel": "decode_split_kernel + decode_combine_kernel (gqa_attn_decode)",
                     "bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_step": win_bytes},
    }
    if pre_ev is not None:
        pre_us = pre_ev[0].elapsed_time(pre_ev[1]) * 1e3
        flops = 4 * w.n_head * w.hd_kv * (n_past * (n_past + 1) // 2) * w.n_layer
        result["prefill_stack"] = {"what": f"append + prefill of {n_past} tokens, {w.n_layer} layers",
                                   "us": round(pre_us, 1),
                                   "attn_tflops_incl_append": round(flops / (pre_us * 1e-6) / 1e12, 2)}
    print(json.dumps(result), flush=True)


def measured_traffic(kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) recorded in
    profiles/ for this workload, or None when the kernel sources changed since the
    counters were taken (the record keeps their sha256)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_qwen3-0.6b-batch.json")
    try:
        rec = json.load(open(path))
        for f, h in rec["source_sha256"].items():
            src = os.path.join(ROOT, "kv_cache_causal_amd", "csrc", f)
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != h:
                return None
        return int(rec[kernel]["fetch_bytes"] + rec[kernel]["write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(orc_cache, w, seqs, lens, kv_bytes, pre_pos, seconds):
    """The oracle, as it stands, on the host cores (plain C, -O2, no FMA, OpenMP over
    independent (token, head) units), timed on bounded samples of the same work:
      - value: the full 32-sequence decode attention (same windows as the GPU step),
        repeated for about `seconds`, on every host thread;
      - prefill: 256 query tokens spread over the 4,096-token prefill, every host thread;
      - single_thread: one thread on the tiny workload (prefill of 8 + 4 decodes), the
        Qwen2.5-0.5B layer decode at 511, and one Qwen3-0.6B layer (prefill of 511 and
        the decode at 511)."""
    from oracle import OracleCache
    from tests import workloads as W
    threads = orc_cache.o.max_threads()
    log(f"bench: oracle baseline on {threads} threads")
    # The step's appends, with the same inputs the GPU step uses: the 4,096-token
    # continuation of sequence 0 and the 32 decode tokens.
    nt = len(pre_pos)
    qp, kp, vp = W.prefill_qkv(w, nt, 0, 0)
    st, qo = orc_cache.append_rope(0, np.zeros(nt, np.int32), pre_pos, qp, w.n_head, w.hd, kp, vp,
                                   w.base, w.freq_scale, w.style)
    assert st == 0
    q, k, v = W.decode_qkv(w, w.n_seq, 0, 0)
    st, q = orc_cache.append_rope(0, seqs, lens, q, w.n_head, w.hd, k, v, w.base, w.freq_scale,
                                  w.style)
    assert st == 0
    reps, t0 = 0, time.perf_counter()
    while True:
        st, _ = orc_cache.attn_decode(0, seqs, lens, q, w.n_head, w.hd, w.scale)
        assert st == 0
        reps += 1
        dec_el = time.perf_counter() - t0
        if dec_el >= seconds:
            break
    dec_gbs = kv_bytes * reps / dec_el / 1e9

    # Prefill sample.
    idx = np.linspace(0, nt - 1, 256).astype(np.int64)
    flops = 4 * w.n_head * w.hd_kv * int((pre_pos[idx].astype(np.int64) + 1).sum())
    t0 = time.perf_counter()
    st, _ = orc_cache.attn_prefill(0, 0, pre_pos[idx], qo[idx], w.n_head, w.hd, w.scale)
    pre_s = time.perf_counter() - t0
    assert st == 0

    single = {}
    # Tiny workload, whole: append + prefill of 8, then 4 x (append + decode).
    tw = W.TINY
    oc = OracleCache(1, 1, tw.n_head_kv, tw.hd_kv, tw.capacity)
    t0 = time.perf_counter()
    n8 = tw.extra["prefill"]
    q8, k8, v8 = W.prefill_qkv(tw, n8, 0)
    _, q8r = oc.append_rope(0, np.zeros(n8, np.int32), np.arange(n8, dtype=np.int32), q8, tw.n_head,
                            tw.hd, k8, v8, tw.base, tw.freq_scale, tw.style)
    oc.attn_prefill(0, 0, np.arange(n8, dtype=np.int32), q8r, tw.n_head, tw.hd, tw.scale, nthreads=1)
    for stp in range(tw.extra["decode_steps"]):
        qq, kk, vv = W.decode_qkv(tw, 1, stp, 0)
        _, qr = oc.append_rope(0, [0], [n8 + stp], qq, tw.n_head, tw.hd, kk, vv, tw.base,
                               tw.freq_scale, tw.style)
        oc.attn_decode(0, [0], [n8 + stp], qr, tw.n_head, tw.hd, tw.scale, nthreads=1)
    single["tiny_whole_us"] = round((time.perf_counter() - t0) * 1e6, 1)
    oc.close()

    def layer_decode_gbs(lw, n_past):
        oc = OracleCache(1, 1, lw.n_head_kv, lw.hd_kv, lw.capacity)
        k, v = W.fill_rows(lw, 0, 0, 0, n_past)
        oc.append_rope(0, np.zeros(n_past, np.int32), np.arange(n_past, dtype=np.int32), None, 0, 0,
                       k.reshape(n_past, lw.n_head_kv, lw.hd_kv),
                       v.reshape(n_past, lw.n_head_kv, lw.hd_kv), lw.base, lw.freq_scale, lw.style)
        qq, kk, vv = W.decode_qkv(lw, 1, 0, 0)
        _, qr = oc.append_rope(0, [0], [n_past], qq, lw.n_head, lw.hd, kk, vv, lw.base,
                               lw.freq_scale, lw.style)
        nb = (n_past + 1) * 2 * lw.n_head_kv * lw.hd_kv * 4
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            oc.attn_decode(0, [0], [n_past], qr, lw.n_head, lw.hd, lw.scale, nthreads=1)
            reps += 1
        el = time.perf_counter() - t0
        oc.close()
        return round(nb * reps / el / 1e9, 3)

    single["qwen25_layer_decode_gbs"] = layer_decode_gbs(W.QWEN25_LAYER, W.QWEN25_LAYER.extra["n_past"])
    sw = W.QWEN3_STACK
    npre = sw.extra["prefill"]
    single["qwen3_layer_decode_gbs"] = layer_decode_gbs(sw, npre)
    oc = OracleCache(1, 1, sw.n_head_kv, sw.hd_kv, sw.capacity)
    qq, kk, vv = W.prefill_qkv(sw, npre, 0)
    ppos = np.arange(npre, dtype=np.int32)
    _, qr = oc.append_rope(0, np.zeros(npre, np.int32), ppos, qq, sw.n_head, sw.hd, kk, vv, sw.base,
                           sw.freq_scale, sw.style)
    t0 = time.perf_counter()
    oc.attn_prefill(0, 0, ppos, qr, sw.n_head, sw.hd, sw.scale, nthreads=1)
    el = time.perf_counter() - t0
    oc.close()
    single["qwen3_layer_prefill_gflops"] = round(4 * sw.n_head * sw.hd_kv * npre * (npre + 1) // 2
                                                 / el / 1e9, 3)
    return {
        "value": round(dec_gbs, 3),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"decode attention of all 32 sequences ({kv_bytes / 1e9:.3f} GB of K/V per "
                  f"pass), {reps} passes in {dec_el:.1f}s on {threads} threads",
        "prefill": {"gflops": round(flops / pre_s / 1e9, 3), "threads": int(threads),
                    "sample": f"256 of the 4096 prefill tokens (every 16th), {flops / 1e9:.2f} "
                              f"GFLOP in {pre_s:.2f}s"},
        "single_thread": single,
    }


if __name__ == "__main__":
    main()
