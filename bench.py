#!/usr/bin/env python3
"""Throughput of the H2O hot path on one MI355X.

One benchmark step is one pass of the whole path over one batch: for every
layer cache, clear it, score and select the prompt (prefill), then run all
decode steps (attention + score accumulation + one eviction + insert per
step). Several independent layer caches are decoded in rotation, token step
by token step, as a model's layers would be, so that no cache is re-read out
of the 256 MB Infinity Cache between its own steps. Inputs are synthetic and
resident in HBM before the timed region starts.

Prints ONE JSON line. ``value`` is decode head-steps per second over the
whole step (prefill included); the roofline object grades the dominant
kernel (the fused decode step) against the 8 TB/s HBM peak; the CPU baseline
is the fp64 oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA peak, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak, TFLOP/s (fp32 prompts run on the VALU)
METRIC = "H2O decode head-steps/sec + achieved HBM GB/s (% of MI355X peak)"
DECODE_SOURCES = {"fused": ["decode.hip", "h2o_device.h", "launch.h"],
                  "split": ["decode_split.hip", "h2o_device.h", "launch.h"],
                  "u8": ["decode_quant.hip", "lane_codes.h", "h2o_device.h", "launch.h"],
                  "u4": ["decode_quant.hip", "lane_codes.h", "h2o_device.h", "launch.h"],
                  "u2": ["decode_quant.hip", "lane_codes.h", "h2o_device.h", "launch.h"]}
QUANT_BITS = {"u8": 8, "u4": 4, "u2": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="opt6.7b_layer")
    p.add_argument("--layers", type=int, default=4, help="independent layer caches decoded in rotation")
    p.add_argument("--decode-steps", type=int, default=None,
                   help="decode steps per bench step (default: the workload's own count; for profiling runs)")
    p.add_argument("--batch", type=int, default=None, help="override the workload's batch")
    p.add_argument("--heads", type=int, default=None, help="override the workload's heads")
    p.add_argument("--prompt-len", type=int, default=None, help="override the workload's prompt length")
    p.add_argument("--decode", choices=("fused", "split"), default="fused",
                   help="decode entry point: h2o_decode_step (fused) or h2o_decode_step_split")
    p.add_argument("--chunk-rows", type=int, default=0, help="split decode chunk length (0 = library's choice)")
    p.add_argument("--prefill", choices=("select", "attention"), default="select",
                   help="prefill entry point: h2o_prefill_select, or h2o_prefill_attention (also returns the "
                        "prompt's attention output)")
    p.add_argument("--quant", choices=("none", "u8", "u4", "u2"), default="none",
                   help="cache storage: rows in the workload dtype, or 8-, 4- or 2-bit codes "
                        "(h2o_cache_init_quant)")
    p.add_argument("--cpu-heads", type=int, default=0,
                   help="heads in the CPU-oracle sample (0: enough for about 15 s of oracle work)")
    p.add_argument("--graph", action="store_true",
                   help="time the step as two captured HIP graphs (clear + prefill of every layer, then the decode "
                        "steps) replayed on the stream, instead of launching each call")
    p.add_argument("--policy", choices=("accumulated", "averaged", "position"), default="accumulated",
                   help="retention value of a slot: accumulated attention (H2O), averaged attention, or position "
                        "(sinks + window)")
    p.add_argument("--k-heavy", type=int, default=None, help="override the workload's k_heavy (0: recent window only)")
    p.add_argument("--k-recent", type=int, default=None,
                   help="override the workload's k_recent (0: heavy hitters only, the new token competes)")
    p.add_argument("--fullcache", action="store_true",
                   help="also time a no-eviction decode attention over the full final length (prompt + decode "
                        "steps) on the same inputs (always on for large_batch_f16)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-single-layer", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run a plain 1 GiB device copy first (scale factor for HBM counters)")
    return p.parse_args()


def decode_source_digest(mode: str = "fused") -> str:
    h = hashlib.sha256()
    for f in DECODE_SOURCES[mode]:
        with open(os.path.join(ROOT, "kv_cache_eviction_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def decode_bytes_per_head(n_used: int, d: int, e: int) -> int:
    """Algorithmic HBM bytes of one fused decode step for one (batch, head).

    reads: K and V rows of the occupied slots, score and pos of every
    occupied slot, q, k_new, v_new; writes: every occupied score, the output
    row (fp32), the new K and V rows, the new slot's pos, the evicted position.
    """
    return 2 * n_used * d * e + 12 * n_used + 5 * d * e + 4 * d + 8


def fullcache_bytes_per_head(length: int, d: int, e: int) -> int:
    """Algorithmic HBM bytes of one no-eviction decode attention for one (batch, head):
    K and V rows of every cached position, the query, the fp32 output row."""
    return 2 * length * d * e + d * e + 4 * d


def decode_bytes_per_head_quant(n_used: int, d: int, e: int, bits: int) -> int:
    """The same for a cache of bits-wide codes: packed codes instead of rows
    (d * bits / 8 bytes each), plus the value grid of every occupied slot and
    the head's key grids; the new token's codes and value grid are written."""
    rb = d * bits // 8
    return 2 * n_used * rb + 8 * n_used + 12 * n_used + 3 * d * e + 8 * d + 4 * d + 2 * rb + 8 + 8


def load_traffic(workload: str, digest: str, mode: str = "fused"):
    name = f"decode_{workload}" if mode == "fused" else f"decode_{mode}_{workload}"
    path = os.path.join(ROOT, "profiles", f"{name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_sample_heads(wl, seconds: float = 15.0) -> int:
    """Heads whose oracle prefill and decode take about `seconds` on 16 host
    threads (per-head cost measured on the OPT-6.7B layer with the oracle's
    heads on 16 threads: 7.3 ps per n^2 d of prefill, 0.30 ns per step x slot
    x channel of decode)."""
    per_head = 7.3e-12 * wl.prompt_len ** 2 * wl.head_dim + 3.0e-10 * wl.steps * wl.k * wl.head_dim
    return int(max(1, min(wl.n_heads_total, round(seconds / per_head))))


def cpu_baseline(wl, heads: int, policy: str = "accumulated"):
    """The fp64 oracle on a bounded sample: `heads` heads, prefill plus every decode step.

    The oracle runs as it stands, evaluating independent heads on one thread
    per CPU this process may use (BLAS single-threaded inside them)."""
    import numpy as np
    from oracle import H2OOracle
    from workload import make_decode, make_prompt, sample_heads

    cores = len(os.sched_getaffinity(0))
    sample = sample_heads(wl, heads or cpu_sample_heads(wl), seed=11)
    Q, K, V = make_prompt(wl, heads=sample)
    q, k, v = make_decode(wl, heads=sample)
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    orc = H2OOracle(sample.size, wl.head_dim, wl.k_heavy, wl.k_recent, wl.scale, policy, workers=cores)
    t0 = time.perf_counter()
    orc.prefill(Q, K, V)
    t1 = time.perf_counter()
    for t in range(wl.steps):
        orc.decode_step(q[:, t], k[:, t], v[:, t])
    t2 = time.perf_counter()
    del np
    return {
        "value": sample.size * wl.steps / (t2 - t0),
        "unit": "head-steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{sample.size} of {wl.n_heads_total} heads, full prompt {wl.prompt_len} prefill + "
                   f"{wl.steps} decode steps, fp64 numpy on {cores} threads over heads "
                   f"(prefill {t1 - t0:.2f} s, decode {t2 - t1:.2f} s)"),
        "decode_only_head_steps_per_s": sample.size * wl.steps / (t2 - t1),
        "prefill_only_heads_per_s": sample.size / (t1 - t0),
        "blas_threads": blas_threads,
    }


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the H2O path shards by (batch, head) with no communication, so a multi-GPU run "
              "is the same kernel on each GPU's share; this benchmark measures one GPU only.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_eviction_decode_amd import H2OCache, load_library
    from kv_cache_eviction_decode_amd.build import ensure_built
    from workload import ELEM_BYTES, WORKLOADS, make_decode, make_prompt

    ensure_built()  # builds only if no build of the current sources exists
    lib = load_library()
    wl = WORKLOADS[args.workload]
    if args.decode_steps is not None:
        wl = wl.with_(steps=max(1, min(args.decode_steps, wl.steps)))
    if args.batch is not None or args.heads is not None:
        wl = wl.with_(batch=args.batch or wl.batch, heads=args.heads or wl.heads)
    if args.prompt_len is not None:
        wl = wl.with_(prompt_len=args.prompt_len)
    if args.k_heavy is not None or args.k_recent is not None:
        wl = wl.with_(k_heavy=wl.k_heavy if args.k_heavy is None else args.k_heavy,
                      k_recent=wl.k_recent if args.k_recent is None else args.k_recent)
    policy = {"accumulated": 0, "averaged": 1, "position": 2}[args.policy]
    default_shape = (args.batch is None and args.heads is None and args.prompt_len is None and args.k_heavy is None
                     and args.k_recent is None and args.policy == "accumulated")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    B, H, d, n, T, L = wl.batch, wl.heads, wl.head_dim, wl.prompt_len, wl.steps, args.layers
    G, k, e = wl.n_heads_total, wl.k, ELEM_BYTES[wl.dtype]
    log(f"[bench] {wl.describe()}; {L} layer caches")

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x 1 GiB device copies done")

    t_gen = time.perf_counter()
    Qh, Kh, Vh = make_prompt(wl)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(tdt)
    Q, K, V = (up(x).view(B, H, n, d) for x in (Qh, Kh, Vh))
    del Qh, Kh, Vh
    qh, kh, vh = make_decode(wl)
    qs, ks, vs = (up(x.transpose(1, 0, 2)).view(T, B, H, d) for x in (qh, kh, vh))
    del qh, kh, vh
    log(f"[bench] inputs generated and resident in HBM ({time.perf_counter() - t_gen:.1f} s)")

    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    quant = args.quant != "none"
    if quant and args.decode == "split":
        raise SystemExit("the split decode entry point takes caches stored in their dtype only")
    caches = [H2OCache(B, H, d, wl.k_heavy, wl.k_recent, tdt, wl.scale, dev, quant=args.quant if quant else None)
              for _ in range(L)]
    qcode = {"u8": 1, "u4": 2, "u2": 3}.get(args.quant, 0)
    ws = caches[0].workspace(n)
    attn = args.prefill == "attention"
    prompt_out = torch.empty(B, H, n, d, dtype=torch.float32, device=dev) if attn else None
    outs = [torch.empty(B, H, d, dtype=torch.float32, device=dev) for _ in range(L)]
    evs = [torch.empty(B, H, dtype=torch.int32, device=dev) for _ in range(L)]
    qp = [qs[t].data_ptr() for t in range(T)]
    kp = [ks[t].data_ptr() for t in range(T)]
    vp = [vs[t].data_ptr() for t in range(T)]
    dcode = {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype]
    split = args.decode == "split"
    sws = caches[0].split_workspace() if split else None  # shared: calls are serialised on one stream

    def check(st):
        if st != 0:
            raise RuntimeError(lib.h2o_last_error().decode())

    def run_prefill(layers, h):
        """Clear and prefill (score, select, gather) the `layers` caches."""
        for i in layers:
            c = caches[i]
            if quant:
                check(lib.h2o_cache_init_quant(ctypes.byref(c.desc), B, H, d, wl.k_heavy, wl.k_recent, policy, dcode,
                                               ctypes.c_float(wl.scale), qcode, c.K.data_ptr(), c.V.data_ptr(),
                                               c.k_qparam.data_ptr(), c.v_qparam.data_ptr(),
                                               c.score.data_ptr(), c.pos.data_ptr(), h))
            else:
                check(lib.h2o_cache_init(ctypes.byref(c.desc), B, H, d, wl.k_heavy, wl.k_recent, policy, dcode,
                                         ctypes.c_float(wl.scale), c.K.data_ptr(), c.V.data_ptr(),
                                         c.score.data_ptr(), c.pos.data_ptr(), h))
            if attn:
                check(lib.h2o_prefill_attention(ctypes.byref(c.desc), Q.data_ptr(), K.data_ptr(), V.data_ptr(), n,
                                                ws.data_ptr(), ws.numel(), prompt_out.data_ptr(), None, None, h))
            else:
                check(lib.h2o_prefill_select(ctypes.byref(c.desc), Q.data_ptr(), K.data_ptr(), V.data_ptr(), n,
                                             ws.data_ptr(), ws.numel(), None, h))

    def run_decode(layers, h):
        """T decode steps, the `layers` caches in rotation token by token."""
        for t in range(T):
            for i in layers:
                if split:
                    check(lib.h2o_decode_step_split(ctypes.byref(caches[i].desc), qp[t], kp[t], vp[t],
                                                    outs[i].data_ptr(), evs[i].data_ptr(), args.chunk_rows,
                                                    sws.data_ptr(), sws.numel(), h))
                else:
                    check(lib.h2o_decode_step(ctypes.byref(caches[i].desc), qp[t], kp[t], vp[t],
                                              outs[i].data_ptr(), evs[i].data_ptr(), h))

    def run_step(layers, ev=None):
        """Whole path for `layers` caches: clear, prefill, T decode steps."""
        run_prefill(layers, sh)
        if ev is not None:
            ev.record(stream)
        run_decode(layers, sh)

    all_layers = list(range(L))
    for _ in range(args.warmup):
        run_step(all_layers)
    torch.cuda.synchronize()

    if args.graph:
        # Capture once: the descriptors' host counters advance during capture,
        # and every replay of the pair restarts from the cleared caches.
        gstream = torch.cuda.Stream()
        gh = ctypes.c_void_p(gstream.cuda_stream)
        g_pre, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(gstream):
            with torch.cuda.graph(g_pre, stream=gstream):
                run_prefill(all_layers, gh)
            with torch.cuda.graph(g_dec, stream=gstream):
                run_decode(all_layers, gh)
        torch.cuda.synchronize()
        # The replayed step must give what the launched step gives.
        run_step(all_layers)
        torch.cuda.synchronize()
        ref = [(x.clone(), y.clone()) for x, y in zip(outs, evs)]
        g_pre.replay()
        g_dec.replay()
        torch.cuda.synchronize()
        for (g_out, g_ev), (r_out, r_ev) in zip(zip(outs, evs), ref):
            if not (torch.equal(g_out, r_out) and torch.equal(g_ev, r_ev)):
                raise RuntimeError("graph replay differs from the launched step")
        for _ in range(max(1, args.warmup)):
            g_pre.replay()
            g_dec.replay()
        torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for s in range(args.steps):
        starts[s].record(stream)
        if args.graph:
            g_pre.replay()
            mids[s].record(stream)
            g_dec.replay()
        else:
            run_step(all_layers, mids[s])
        ends[s].record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - w0
    step_ms = [starts[s].elapsed_time(ends[s]) for s in range(args.steps)]
    prefill_ms = [starts[s].elapsed_time(mids[s]) for s in range(args.steps)]
    decode_ms = [mids[s].elapsed_time(ends[s]) for s in range(args.steps)]
    # Every figure is the median over the timed steps (the mean is reported beside it).
    median = lambda xs: float(np.median(np.asarray(xs, dtype=np.float64)))
    ms_per_step = median(step_ms)
    head_steps = G * T * L
    value = head_steps / (ms_per_step / 1e3)

    n_used = [min(k, n + t) for t in range(T)]
    if quant:
        bits = QUANT_BITS[args.quant]
        bytes_per_launch = G * sum(decode_bytes_per_head_quant(u, d, e, bits) for u in n_used) / T
    else:
        bytes_per_launch = G * sum(decode_bytes_per_head(u, d, e) for u in n_used) / T
    launches = T * L
    avg_launch_s = median(decode_ms) / 1e3 / launches
    achieved = bytes_per_launch / avg_launch_s / 1e9
    mode = args.quant if quant else args.decode
    # the library runs one wave per head when the heads fill half the resident waves (2 per SIMD)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    fused_kernel = "decode_wave_kernel" if G >= cus * 4 else "decode_kernel"
    quant_kernel = "decode_quant_kernel" if G >= cus * 4 else "decode_quant_wg_kernel"
    digest = decode_source_digest(mode)
    traffic = load_traffic(wl.name, digest, mode) if default_shape else None
    # two causal QK^T passes per layer (d n (n+1) flops each), plus the causal P.V with the output
    prefill_flops = (3.0 if attn else 2.0) * n * (n + 1) * d * G
    pf_s = median(prefill_ms) / 1e3 / L

    single = None
    if not args.no_single_layer and L > 1:
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for s in range(2):
            e0[s].record(stream)
            run_step([0], e1[s])
        e2 = torch.cuda.Event(enable_timing=True)
        e2.record(stream)
        torch.cuda.synchronize()
        dms = e1[1].elapsed_time(e2)
        single = {"decode_us_per_launch": dms * 1e3 / T,
                  "decode_GBps": bytes_per_launch / (dms / 1e3 / T) / 1e9,
                  "note": f"one cache decoded alone: its {bytes_per_launch / 1e6:.0f} MB per step can be partly "
                          "re-read from the 256 MB Infinity Cache"}

    # Secondary denominator: what a plain device-to-device copy of 1 GiB
    # moves per second on this GPU (bytes read + bytes written).
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    for _ in range(2):
        cdst.copy_(csrc)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (c0.elapsed_time(c1) / 1e3) / 1e9
    del csrc, cdst

    fullcache = None
    if args.fullcache or wl.name == "large_batch_f16":
        # The comparator of the large-batch workload: the same step without
        # eviction, i.e. plain decode attention over every position of the
        # final length, with the same prompt and decode keys/values.
        from kv_cache_eviction_decode_amd import h2o_fullcache_decode
        Lf = n + T
        Kc = torch.cat([K, ks.permute(1, 2, 0, 3)], dim=2).contiguous()
        Vc = torch.cat([V, vs.permute(1, 2, 0, 3)], dim=2).contiguous()
        fout = torch.empty(B, H, d, dtype=torch.float32, device=dev)
        reps = 20
        for _ in range(3):
            h2o_fullcache_decode(qs[T - 1], Kc, Vc, fout, wl.scale, stream)
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(reps):
            h2o_fullcache_decode(qs[T - 1], Kc, Vc, fout, wl.scale, stream)
        f1.record(stream)
        torch.cuda.synchronize()
        f_s = f0.elapsed_time(f1) / 1e3 / reps
        f_bytes = G * fullcache_bytes_per_head(Lf, d, e)
        h2o_full_bytes = G * decode_bytes_per_head(k, d, e)
        fullcache = {"kernel": "h2o decode_wave_kernel, unscored mode (no scores, no eviction)",
                     "length": Lf, "us_per_launch": f_s * 1e6, "head_steps_per_s": G / f_s,
                     "GBps": f_bytes / f_s / 1e9, "hbm_frac": f_bytes / f_s / 1e9 / HBM_PEAK_GBS,
                     "bytes_per_launch": f_bytes,
                     "h2o_bytes_per_launch_full_cache": h2o_full_bytes,
                     "bytes_ratio_fullcache_over_h2o": f_bytes / h2o_full_bytes,
                     "h2o_avg_launch_us": avg_launch_s * 1e6,
                     "time_ratio_fullcache_over_h2o": f_s / avg_launch_s,
                     "note": f"{reps} launches over a {Lf}-position cache after 3 warm-up launches, query of the "
                             "last decode step; H2O bytes are those of a full k-slot step"}
        del Kc, Vc

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_mean": sum(step_ms) / args.steps,
        "timing": f"median of {args.steps} timed steps after {args.warmup} warm-up steps (HIP events)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "heads": H, "head_dim": d, "prompt_len": n,
                   "k_heavy": wl.k_heavy, "k_recent": wl.k_recent, "decode_steps": T, "layers": L,
                   "pareto_alpha": wl.alpha, "parallelism": "none (1 GPU)", "decode_entry": args.decode,
                   "cache_storage": f"{args.quant} codes" if quant else wl.dtype, "policy": args.policy,
                   "launch": "graph" if args.graph else "eager"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": ("h2o decode_chunk_kernel + decode_merge_kernel (split decode)" if split else
                                f"h2o {quant_kernel} (fused step over {args.quant} codes)" if quant else
                                f"h2o {fused_kernel} (fused attention + score + evict + insert)"),
                     "bytes_per_launch": bytes_per_launch, "avg_launch_us": avg_launch_s * 1e6,
                     "kernel_source_digest": digest,
                     "library_digest": lib.h2o_build_digest().decode(),
                     "copy_GBps": copy_gbps, "frac_of_copy": achieved / copy_gbps,
                     "copy_note": "plain 1 GiB device-to-device copy (read + write bytes), 5 timed"},
        "decode_head_steps_per_s": head_steps / (median(decode_ms) / 1e3),
        "prefill": {"ms_per_layer": pf_s * 1e3, "algorithmic_TFLOPs": prefill_flops / pf_s / 1e12,
                    "mfma_frac": (prefill_flops / pf_s / 1e12 / MFMA_BF16_PEAK_TFLOPS) if wl.dtype != "f32" else None,
                    "bound": "mfma" if wl.dtype != "f32" else "valu",
                    "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS if wl.dtype != "f32" else FP32_VECTOR_PEAK_TFLOPS,
                    "frac": prefill_flops / pf_s / 1e12 /
                            (MFMA_BF16_PEAK_TFLOPS if wl.dtype != "f32" else FP32_VECTOR_PEAK_TFLOPS),
                    # one causal QK^T pass is the least any exact column sum needs
                    "one_pass_TFLOPs": 1.0 * n * (n + 1) * d * G / pf_s / 1e12,
                    # exp2 per score in each pass: n(n+1)/2 per head and pass
                    "exp_per_layer": float(n) * (n + 1) * G, "exp_per_s": float(n) * (n + 1) * G / pf_s,
                    "entry": args.prefill,
                    "note": ("rowattn (QK^T + P.V, prompt output) + colsum (QK^T) + select/gather + cache clear"
                             if attn else "rowlse + colsum + select/gather + cache clear, 2 causal QK^T passes")},
        "wall_s_timed": wall_s,
        "single_layer": single,
        "fullcache": fullcache,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_heads, args.policy)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
