#!/usr/bin/env python3
"""Benchmark of one attention layer's engine step on one MI355X.

A timed step is the whole hot path over one synthetic batch:
  a1  C++ FIFO builder step (the builder state restored from a snapshot of
      the prepared state first, so every timed step is the same step),
  a2  the descriptor packed into pinned memory and uploaded in one async copy,
  a3  cb_kv_append of the step's K/V rows,
  a4-a7  cb_attention_step (plan, the ragged decode+prefill kernel, split-K
      combine, bf16 output).
The default workload is the mixed step: 64 decode sequences (context uniform
on [256, 8192]) plus prefill chunks 476 (at offset 1024), 700 and 808 of
three prompts under max_batch_tokens = 2048; 32 query / 8 KV heads, head_dim
128, bf16, 16-token pages.  ``--workload`` selects the other shapes.

Prints ONE JSON line on stdout: query tokens/s, ms per step, the roofline of
the main attention kernel (its duration measured with HIP events recorded on
its stream around each launch), and the CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import json
import subprocess
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
MFMA_F32_PEAK_TFLOPS = 157.3

METRIC = "query tokens/s per mixed attention step + % of HBM/MFMA roofline, 1 MI355X"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording
    it writes a timestamp without the system-scope cache writeback and
    invalidation a default event performs (which costs the following kernels
    a few microseconds each).  Same use as torch.cuda.Event(enable_timing=True);
    the handle goes to the library's profiling hooks as is."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch and libcb already share
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._h = ctypes.c_void_p()
        if TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._h), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    @property
    def cuda_event(self):
        return self._h.value

    def record(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        if TimingEvent._hip.hipEventRecord(self._h, s.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        if TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self._h, end._h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._h and TimingEvent._hip is not None:
            TimingEvent._hip.hipEventDestroy(self._h)


class CacheFlush:
    """Empties the L2 and Infinity Cache of a step's data before a cold step.

    write: every byte of a 1 GiB buffer is written (the dirty lines it leaves
    are written back while the next step evicts them, so that step also pays
    up to the caches' size in extra HBM writes).  read: a 1 GiB buffer,
    written once here, is read through by a sum; the caches then hold only
    clean lines of unrelated data, and the step's own traffic is all it
    moves."""

    def __init__(self, mode, dev):
        import torch
        self.mode = mode
        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        self.buf.fill_(1)
        self.acc = torch.zeros((), dtype=torch.int64, device=dev)

    def __call__(self, k, stream):
        import torch
        with torch.cuda.stream(stream):
            if self.mode == "write":
                self.buf.fill_(k & 255)
            else:
                torch.sum(self.buf.view(torch.int64), dim=0, out=self.acc)


def workload(name):
    import workloads as wl
    if name == "mixed":
        return wl.mixed(), 0
    if name == "decode":
        return wl.decode_only(), 0
    if name == "long":
        return wl.long_prompt(), 38          # the heaviest 512-token chunk (offset 19456)
    if name == "chunk":
        w = wl.long_prompt()
        w.requests = [r for r in w.requests if r[2] == 0]     # the long prompt alone
        w.name = "longprompt_chunk_only_512@19456_gqa64/8_d128_bf16"
        return w, 38
    raise SystemExit(f"unknown workload {name}")


def counted_traffic(workload_name, kernel):
    """HBM bytes per launch of the given kernel from the committed rocprofv3
    counter runs (FETCH_SIZE / WRITE_SIZE scaled by the copy-kernel
    calibration), or None when the kernel source changed since they were taken
    or no record covers this workload and kernel."""
    import glob
    import hashlib
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")):
        rec = json.load(open(path))
        if rec.get("workload") != workload_name or rec.get("kernel") != kernel:
            continue
        src = os.path.join(ROOT, rec["source"])
        if os.path.exists(src) and hashlib.sha256(open(src, "rb").read()).hexdigest() == rec["source_sha256"]:
            return rec["traffic_bytes"]
    return None


def first_held_position(builder, req_id):
    """First logical position of a request whose page the builder holds."""
    import numpy as np
    held = np.nonzero(np.asarray(builder.block_table(req_id)) >= 0)[0]
    return int(held[0]) * 16 if len(held) else 1 << 30


def algorithmic(desc, hq, hkv, d, esize, window=0):
    """Bytes the step must move and flops it must do (no padding, no re-reads).

    With a sliding window a sequence needs the keys from its first row's
    window start on, and row p sees min(p + 1, window) keys."""
    import numpy as np
    ctx = desc.context_lens.astype(np.int64)
    ql = desc.q_lens.astype(np.int64)
    off = ctx - ql
    first = np.maximum(0, off - window + 1) if window > 0 else np.zeros_like(off)
    kv = int(((ctx - first) * 2 * hkv * d * esize).sum())
    qo = int(2 * desc.num_tokens * hq * d * esize)
    meta = int((-(-ctx // 16) - first // 16).sum() * 4 + (3 * desc.num_seqs + 1) * 4)
    if window > 0:
        pairs = np.array([int(np.minimum(np.arange(o + 1, c + 1), window).sum()) for o, c in zip(off, ctx)],
                         dtype=np.int64)
    else:
        pairs = ql * off + ql * (ql + 1) // 2
    flops = int((4 * d * hq * pairs).sum())
    return kv + qo + meta, flops, int(pairs.sum()), kv


def prepare_layer(w, args, dev, gq=0, gkv=0):
    """The workload's engine layer with every request submitted and its cached
    history imported; returns the layer and the per-request K/V histories."""
    from chunked_prefill_attention_amd.engine import PagedAttentionLayer
    import workloads as wl
    hkv, d = w.n_kv_heads, w.head_dim
    layer = PagedAttentionLayer(w.n_q_heads, hkv, d, w.pool_pages, w.max_batch_tokens, w.max_requests, w.dtype,
                                w.max_prefill_chunk, w.safety_margin,
                                page_shuffle_seed=w.seed if args.page_order == "shuffled" else 0, device=dev,
                                sliding_window=args.window, graph_q_interval=gq, graph_kv_interval=gkv)
    hist = {}
    for i, (p, o, c) in enumerate(w.requests):
        layer.builder.submit(i, p, o, c)
    # K/V histories drawn on the device, per request (exact bf16 values)
    for i, (p, o, c) in enumerate(w.requests):
        n = p + o - 1
        k = wl.device_normal((n, hkv, d), w.dtype, dev, w.seed, i, 1)
        v = wl.device_normal((n, hkv, d), w.dtype, dev, w.seed, i, 2)
        hist[i] = (k, v)
        # the cached history the builder holds pages for (under a sliding
        # window, pages wholly below the next row's window are not held)
        lo = min(first_held_position(layer.builder, i), c)
        if lo < c:
            layer.write_positions(i, lo, c, k[lo:c], v[lo:c])
    return layer, hist


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed", choices=["mixed", "decode", "long", "chunk", "trace"],
                    help="trace: the 256-request FIFO trace run once, every step timed cold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace-csv", default="", help="trace workload and --sweep: also write one CSV row per step here")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle leg")
    ap.add_argument("--page-order", default="shuffled", choices=["shuffled", "sequential"],
                    help="physical page ids: a seeded random permutation (default) or handed out in order")
    ap.add_argument("--graphs", default="",
                    help="Q,KV padding intervals: replay each padded step shape from a recorded HIP graph")
    ap.add_argument("--cold", default="auto", choices=["auto", "on", "off"],
                    help="empty the caches (1 GiB written or read, --flush) before every timed step so that no cache level holds "
                         "the step's data (auto: on when the step moves less than 1 GB); the step time is then "
                         "the device span of each step")
    ap.add_argument("--flush", default="read", choices=["read", "write"],
                    help="how a cold step's caches are emptied: write 1 GiB (its dirty lines are written back "
                         "during the step) or read 1 GiB (clean lines only)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock measurement of MFMA-bound steps (40 extra back-to-back calls)")
    ap.add_argument("--sweep", action="store_true",
                    help="long / chunk workloads: time every step that carries a chunk of the 20,000-token "
                         "prompt (40 steps), each --steps times cold after --warmup untimed runs")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in tokens (row p sees keys p-W < j <= p); 0 = full attention")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here "
              "(the attention step would shard by sequence or by KV head, with no exchange between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import chunked_prefill_attention_amd as cb
    import workloads as wl

    if args.sweep and args.workload not in ("long", "chunk"):
        raise SystemExit("--sweep applies to the long and chunk workloads")
    cb.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.workload == "trace":
        return run_trace(args, dev)
    w, advance = workload(args.workload)
    if args.window > 0:
        w.name += f"_window{args.window}"
    if args.sweep:
        return run_sweep(args, dev, w)
    gq, gkv = (int(x) for x in args.graphs.split(",")) if args.graphs else (0, 0)
    hq, hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
    t_setup = time.perf_counter()
    layer, hist = prepare_layer(w, args, dev, gq, gkv)
    for _ in range(advance):                       # earlier steps: append only
        desc = layer.schedule()
        ks = torch.cat([hist[int(r)][0][a:e] for r, a, e in zip(desc.req_ids, desc.q_offsets, desc.context_lens)])
        vs = torch.cat([hist[int(r)][1][a:e] for r, a, e in zip(desc.req_ids, desc.q_offsets, desc.context_lens)])
        cb.kv_append(ks, vs, layer.k_cache, layer.v_cache, torch.from_numpy(desc.slot_mapping).to(dev))
    snapshot = layer.builder.clone()               # the step's starting state
    desc0 = layer.schedule().copy()
    T = desc0.num_tokens
    q = wl.device_normal((T, hq, d), w.dtype, dev, w.seed, 99, 3)
    kn = torch.cat([hist[int(r)][0][a:e] for r, a, e in zip(desc0.req_ids, desc0.q_offsets, desc0.context_lens)])
    vn = torch.cat([hist[int(r)][1][a:e] for r, a, e in zip(desc0.req_ids, desc0.q_offsets, desc0.context_lens)])
    out = torch.empty_like(q)
    layer.attend(q, kn, vn, out=out)               # sizes the workspace
    torch.cuda.synchronize()
    if layer.graphs:                               # the step's inputs live in the static buffers
        layer.static_q[:T].copy_(q)
        layer.static_k[:T].copy_(kn)
        layer.static_v[:T].copy_(vn)
        q, kn, vn, out = layer.static_q, layer.static_k, layer.static_v, layer.static_out
        torch.cuda.synchronize()
    log(f"[bench] {w.name}: setup {time.perf_counter() - t_setup:.1f}s; step: {desc0.num_seqs} seqs, "
        f"{desc0.num_decodes} decodes, {T} query tokens, max ctx {desc0.max_context_len}")

    esize = 2 if w.dtype == "bf16" else 4
    bytes_alg, flops_alg, pairs, kv_alg = algorithmic(desc0, hq, hkv, d, esize, args.window)
    lib = cb.load()
    cold = args.cold == "on" or (args.cold == "auto" and bytes_alg < 1e9)
    flush = CacheFlush(args.flush, dev) if cold else None
    starts = [TimingEvent() for _ in range(args.steps)]
    stops = [TimingEvent() for _ in range(args.steps)]
    span0 = [TimingEvent() for _ in range(args.steps)]
    span1 = [TimingEvent() for _ in range(args.steps)]
    mid0 = [TimingEvent() for _ in range(args.steps)]   # span pass: the main kernel's start and end too
    mid1 = [TimingEvent() for _ in range(args.steps)]
    for e in starts + stops + span0 + span1 + mid0 + mid1:
        e.record()
    stream = layer.graph_stream if layer.graphs else torch.cuda.current_stream(dev)

    def one_step(k=None, flush_first=True, span=None):
        if cold and flush_first:                               # evict the step's data from L2 and MALL
            flush(k or 0, stream)
        layer.load_builder(snapshot)                           # same starting state each time
        layer.schedule(stream=stream)                          # a1 + a2
        if layer.graphs:                                       # events around the whole graph
            if k is not None:
                starts[k].record(stream)
            layer._attend(q, kn, vn, out, stream)              # a3 .. a7, replayed
            if k is not None:
                stops[k].record(stream)
            return
        if k is not None:     # timed steps: events around the main kernel only
            lib.cb_profile_events(starts[k].cuda_event, stops[k].cuda_event)
        elif span is not None:  # the span pass: events around the whole step and the main kernel
            span0[span].record(stream)
            lib.cb_profile_events(mid0[span].cuda_event, mid1[span].cuda_event)
        layer.attend(q, kn, vn, out=out, stream=stream)        # a3 .. a7
        if k is not None:
            lib.cb_profile_events(None, None)
        elif span is not None:
            lib.cb_profile_events(None, None)
            span1[span].record(stream)

    for i in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(k)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, stops)]
    kern_s = float(np.mean(kern_ms)) / 1e3
    if layer.graphs:      # the graph's events already span append .. combine
        span_ms = kern_ms
    else:                 # a second pass of as many steps, events around each whole step
        for k in range(args.steps):
            one_step(span=k)
        torch.cuda.synchronize()
        span_ms = [s.elapsed_time(e) for s, e in zip(span0, span1)]
        # the step's other launches: append (with the metadata pull) before the
        # main kernel, combine after it, each with its launch gap
        append_us = float(np.mean([s.elapsed_time(m) for s, m in zip(span0, mid0)])) * 1e3
        combine_us = float(np.mean([m.elapsed_time(e) for m, e in zip(mid1, span1)])) * 1e3
    span_s = float(np.mean(span_ms)) / 1e3
    if cold:              # the wall clock includes the flushes: a step is its device span
        step_s = span_s
    assert torch.isfinite(out[:T].float()).all(), "non-finite attention output"

    t_hbm, t_mfma = bytes_alg / (HBM_PEAK_GBS * 1e9), flops_alg / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(bytes_alg / kern_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(bytes_alg / kern_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(flops_alg / kern_s / 1e12, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(flops_alg / kern_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    kname = "attn_mixed_kernel" if desc0.num_seqs > desc0.num_decodes else "attn_decode_kernel"
    roof["kernel"] = f"{kname}<{d}, {'true' if args.window > 0 else 'false'}>"   # the template instance timed
    roof["traffic"] = counted_traffic(w.name, roof["kernel"])
    if layer.graphs:
        roof["kernel"] = "graph replay (kv_append + attention + combine)"
        roof["traffic"] = None
        roof["graphs"] = layer.graph_stats()
    roof["kernel_us"] = round(kern_s * 1e6, 2)
    roof["step_roofline_frac"] = round(max(t_hbm, t_mfma) / step_s, 4)
    roof["device_span_us"] = round(span_s * 1e6, 2)   # kv_append .. combine on the device
    if not layer.graphs:
        roof["append_us"] = round(append_us, 2)        # kv_append (+ metadata pull), up to the main kernel
        roof["combine_us"] = round(combine_us, 2)      # after the main kernel: split-K combine
    pct = lambda xs, q: round(float(np.percentile(xs, q)) * 1e3, 2)
    roof["kernel_us_p10_p50_p90"] = [pct(kern_ms, 10), pct(kern_ms, 50), pct(kern_ms, 90)]
    roof["span_us_p10_p50_p90"] = [pct(span_ms, 10), pct(span_ms, 50), pct(span_ms, 90)]
    roof["timing"] = (f"cold: 1 GiB {'written' if args.flush == 'write' else 'read'} before each step; "
                      "step = device span" if cold
                      else "warm: steps back to back; step = wall time; HIP events around the main kernel only "
                           "(the device span from a second pass with events around each step)")
    if roof["bound"] == "mfma" and not args.no_clock:  # the shader clock the chip holds under this load
        # the step's attention called back to back on its own descriptor (the
        # host enqueues far faster than the kernel runs, so the chip stays busy)
        dq = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev) for a in
              (desc0.block_tables, desc0.query_start_loc, desc0.context_lens, desc0.q_offsets)]
        ws = torch.empty(max(cb.attention_workspace_bytes(desc0.num_seqs, desc0.num_decodes, T, hq, hkv, d,
                                                          desc0.max_context_len, cb.CB_BF16), 1),
                         dtype=torch.uint8, device=dev)
        o2 = torch.empty_like(q[:T])

        def attention_burst():
            for _ in range(8):
                cb.attention_step(q[:T], layer.k_cache, layer.v_cache, *dq, desc0.num_decodes, desc0.max_context_len,
                                  layer.scale, out=o2, workspace=ws, stream=stream)
        clk = kernel_clock_mhz(attention_burst, lib, dev)
        roof["clock_mhz"] = clk
        if clk and clk.get("mean"):
            # the same rate against the MFMA peak scaled to the measured clock (the published peak assumes 2.4 GHz)
            roof["frac_at_measured_clock"] = round(roof["frac"] * 2400.0 / clk["mean"], 4)
    if roof["bound"] == "hbm":   # beside the peak: a plain streaming read of as many bytes
        ach = achievable_read_gbs(max(bytes_alg, 1 << 30))
        roof["achievable_read_GBps"] = ach
        roof["frac_of_achievable"] = round(roof["achieved"] / ach, 4) if ach else None
    elif not args.no_clock:      # beside the peak: a plain bf16 GEMM of the vendor BLAS
        ach = achievable_gemm_tflops(dev)
        roof["achievable_gemm_TFLOPs"] = ach
        roof["frac_of_achievable"] = round(roof["achieved"] / ach, 4) if ach else None
    log(f"[bench] host enqueue {(t_enq - t0) / args.steps * 1e3:.3f} ms/step")
    log(f"[bench] device span (append .. combine) {span_s * 1e6:.1f} us")
    log(f"[bench] step {step_s * 1e3:.3f} ms, attention kernel {kern_s * 1e6:.1f} us, "
        f"{bytes_alg / 1e9:.3f} GB algorithmic, {flops_alg / 1e9:.1f} GFLOP")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(desc0, q, hist, hq, hkv, d, args.cpu_seconds, out, args.window)

    rec = {
        "metric": METRIC, "value": round(T / step_s, 1), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V; no dataset)",
        "config": {"workload": w.name, "page_order": args.page_order, "num_seqs": desc0.num_seqs, "num_decodes": desc0.num_decodes,
                   "num_tokens": T, "q_heads": hq, "kv_heads": hkv, "head_dim": d, "page_size": 16,
                   "max_batch_tokens": w.max_batch_tokens, "max_context_len": desc0.max_context_len,
                   "sliding_window": args.window, "graph_padding": [gq, gkv],
                   "algorithmic_bytes": bytes_alg, "algorithmic_kv_bytes": kv_alg,
                   "algorithmic_other_bytes": bytes_alg - kv_alg, "visible_pairs": pairs,
                   "algorithmic_flops": flops_alg},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def run_trace(args, dev):
    """The FIFO trace (256 requests: Poisson arrivals, lognormal prompts,
    geometric outputs; pool 200,000 pages; 64q/8kv, D 128, bf16) run once
    through the engine.  Every step is timed once, cold (1 GiB written or read before
    it), as its device span (append .. combine), and classified HBM- or
    MFMA-bound by its algorithmic bytes and flops."""
    import numpy as np
    import torch
    import chunked_prefill_attention_amd as cb
    from chunked_prefill_attention_amd.engine import PagedAttentionLayer
    import workloads as wl
    hq, hkv, d, dtype, esize = 64, 8, 128, "bf16", 2
    reqs = wl.fifo_trace()
    layer = PagedAttentionLayer(hq, hkv, d, 200_000, 2048, 128, dtype, 0, 0.15, page_shuffle_seed=5, device=dev)
    lib = cb.load()
    stream = torch.cuda.current_stream(dev)
    flush = CacheFlush(args.flush, dev)
    ev = [TimingEvent() for _ in range(4)]
    for e in ev:
        e.record()
    pending, step = list(reqs), 0
    rows = []                          # (tokens, bytes, flops, span_s, kernel_s, class, seqs, decodes, max ctx)
    frag = []
    t0 = time.perf_counter()
    while True:
        st = layer.builder.stats()
        if not pending and st["num_waiting"] + st["num_prefilling"] + st["num_decoding"] \
                + st["num_finished_pending"] == 0:
            break
        while pending and pending[0].arrival_step <= step:
            r = pending.pop(0)
            layer.builder.submit(r.req_id, r.prompt_len, r.output_len)
        desc = layer.schedule()
        step += 1
        if desc.num_tokens == 0:
            continue
        T = desc.num_tokens
        kn = wl.device_normal((T, hkv, d), dtype, dev, 5, step, 1)
        vn = wl.device_normal((T, hkv, d), dtype, dev, 5, step, 2)
        q = wl.device_normal((T, hq, d), dtype, dev, 5, step, 3)
        flush(step, stream)
        ev[0].record(stream)
        lib.cb_profile_events(ev[2].cuda_event, ev[3].cuda_event)
        layer.attend(q, kn, vn, stream=stream)
        lib.cb_profile_events(None, None)
        ev[1].record(stream)
        torch.cuda.synchronize()
        nbytes, flops, _, _ = algorithmic(desc, hq, hkv, d, esize)
        cls = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
        rows.append((T, nbytes, flops, ev[0].elapsed_time(ev[1]) / 1e3, ev[2].elapsed_time(ev[3]) / 1e3, cls,
                     desc.num_seqs, desc.num_decodes, int(desc.context_lens.max())))
        st = layer.builder.stats()
        if st["allocated_slots"]:
            frag.append(st["fragmentation"])
    wall = time.perf_counter() - t0
    if args.trace_csv:
        with open(args.trace_csv, "w") as f:
            f.write("query_tokens,alg_bytes,alg_flops,span_s,kernel_s,class,seqs,decodes,max_ctx\n")
            for r in rows:
                f.write(",".join(str(x) for x in r) + "\n")
    tok = sum(r[0] for r in rows)
    span = sum(r[3] for r in rows)
    classes = {}
    for c in ("hbm", "mfma"):
        sel = [r for r in rows if r[5] == c]
        if not sel:
            continue
        ts, tk = sum(r[3] for r in sel), sum(r[4] for r in sel)
        b, f = sum(r[1] for r in sel), sum(r[2] for r in sel)
        classes[c] = {"steps": len(sel), "query_tokens": sum(r[0] for r in sel), "device_span_s": round(ts, 4),
                      "kernel_s": round(tk, 4),
                      "kernel_frac_of_peak": round((b / tk / 1e9 / HBM_PEAK_GBS) if c == "hbm"
                                                   else (f / tk / 1e12 / MFMA_BF16_PEAK_TFLOPS), 4)}
    top = max(classes, key=lambda c: classes[c]["kernel_s"])
    sel = [r for r in rows if r[5] == top]
    tk = sum(r[4] for r in sel)
    if top == "hbm":
        ach = sum(r[1] for r in sel) / tk / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        ach = sum(r[2] for r in sel) / tk / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof.update({"frac": round(ach / roof["peak"], 4), "traffic": None,
                 "kernel": "attn_mixed_kernel / attn_decode_kernel <128, false> (the trace's steps of this class)"})
    log(f"[bench] trace: {len(rows)} steps, {tok} query tokens, device {span:.3f} s, wall {wall:.1f} s; "
        + ", ".join(f"{c}: {v['steps']} steps {v['kernel_frac_of_peak']:.3f} of peak" for c, v in classes.items()))
    rec = {
        "metric": METRIC, "value": round(tok / span, 1), "unit": "query tokens/s", "n_gpus": 1,
        "steps": len(rows), "warmup": 0, "ms_per_step": round(span / len(rows) * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V; no dataset)",
        "config": {"workload": "fifo_trace_256req_poisson0.5_lognormal1500_geom256_gqa64/8_d128_bf16",
                   "pool_pages": 200_000, "max_batch_tokens": 2048, "max_requests": 128, "safety_margin": 0.15,
                   "timing": f"each step once, cold (1 GiB {'written' if args.flush == 'write' else 'read'} "
                             "before it); step = device span"},
        "roofline": roof,
        "trace": {"query_tokens": tok, "device_span_s": round(span, 4), "classes": classes,
                  "fragmentation_mean": round(float(np.mean(frag)), 5) if frag else None,
                  "fragmentation_max": round(float(np.max(frag)), 5) if frag else None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def run_sweep(args, dev, w):
    """Every step of the long-prompt workload that carries a chunk of its
    20,000-token prompt (40 steps of 512 tokens, the last 32), in order, or,
    with the chunk workload, the same 40 chunks without the decodes.  Each
    step runs --warmup untimed and --steps timed times back to back from the
    same builder state, cold under --cold's rule (by default the steps that move less than
    1 GB); the step's time is the median device span (append .. combine), its
    kernel time the median of HIP events around the main attention kernel.  Each step is classed HBM- or MFMA-bound
    by its algorithmic bytes and flops; the roofline line aggregates the class
    that holds most of the kernel time."""
    import numpy as np
    import torch
    import chunked_prefill_attention_amd as cb
    import workloads as wl
    hq, hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
    esize = 2 if w.dtype == "bf16" else 4
    t_setup = time.perf_counter()
    layer, hist = prepare_layer(w, args, dev)
    lib = cb.load()
    stream = torch.cuda.current_stream(dev)
    flush = CacheFlush(args.flush, dev)
    ev = [[TimingEvent() for _ in range(4)] for _ in range(args.steps)]
    for e in sum(ev, []):
        e.record()
    log(f"[bench] {w.name} sweep: setup {time.perf_counter() - t_setup:.1f}s")
    rows = []
    for k in range(1 << 16):
        snapshot = layer.builder.clone()
        desc = layer.schedule().copy()
        if desc.num_seqs == desc.num_decodes:        # the prompt's last chunk is done
            break
        T = desc.num_tokens
        q = wl.device_normal((T, hq, d), w.dtype, dev, w.seed, 99, 3, k)
        kn = torch.cat([hist[int(r)][0][a:e] for r, a, e in zip(desc.req_ids, desc.q_offsets, desc.context_lens)])
        vn = torch.cat([hist[int(r)][1][a:e] for r, a, e in zip(desc.req_ids, desc.q_offsets, desc.context_lens)])
        out = torch.empty_like(q)
        nbytes, flops, _, _ = algorithmic(desc, hq, hkv, d, esize, args.window)
        cold = args.cold == "on" or (args.cold == "auto" and nbytes < 1e9)
        for r in range(args.warmup + args.steps):       # back to back, as the engine runs steps
            layer.load_builder(snapshot)
            layer.schedule(stream=stream)
            if cold:
                flush(r, stream)
            e = ev[r - args.warmup] if r >= args.warmup else None
            if e:
                e[0].record(stream)
                lib.cb_profile_events(e[2].cuda_event, e[3].cuda_event)
            layer.attend(q, kn, vn, out=out, stream=stream)
            if e:
                lib.cb_profile_events(None, None)
                e[1].record(stream)
        torch.cuda.synchronize()
        span = [e[0].elapsed_time(e[1]) / 1e3 for e in ev]
        kern = [e[2].elapsed_time(e[3]) / 1e3 for e in ev]
        assert torch.isfinite(out.float()).all(), f"non-finite attention output at step {k}"
        cls = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
        ks, ss = float(np.median(kern)), float(np.median(span))
        frac = nbytes / ks / 1e9 / HBM_PEAK_GBS if cls == "hbm" else flops / ks / 1e12 / MFMA_BF16_PEAK_TFLOPS
        pf = int(desc.num_decodes)                   # the prompt's chunk follows the step's decodes
        rows.append({"step": k, "query_tokens": T, "decodes": int(desc.num_decodes),
                     "chunk_offset": int(desc.q_offsets[pf]), "chunk_tokens": int(desc.q_lens[pf]),
                     "alg_bytes": nbytes, "alg_flops": flops, "class": cls, "cold": int(cold),
                     "kernel_us": round(ks * 1e6, 2), "span_us": round(ss * 1e6, 2), "kernel_frac": round(frac, 4)})
        log(f"[bench] step {k}: chunk {rows[-1]['chunk_offset']}+{rows[-1]['chunk_tokens']}, "
            f"{desc.num_decodes} decodes, kernel {ks * 1e6:.1f} us, span {ss * 1e6:.1f} us, {cls} {frac:.3f}")
    if args.trace_csv:
        with open(args.trace_csv, "w") as f:
            f.write(",".join(rows[0]) + "\n")
            for r in rows:
                f.write(",".join(str(v) for v in r.values()) + "\n")
    classes = {}
    for c in ("hbm", "mfma"):
        sel = [r for r in rows if r["class"] == c]
        if not sel:
            continue
        tk = sum(r["kernel_us"] for r in sel) / 1e6
        b, f = sum(r["alg_bytes"] for r in sel), sum(r["alg_flops"] for r in sel)
        classes[c] = {"steps": len(sel), "kernel_s": round(tk, 6),
                      "kernel_frac_of_peak": round((b / tk / 1e9 / HBM_PEAK_GBS) if c == "hbm"
                                                   else (f / tk / 1e12 / MFMA_BF16_PEAK_TFLOPS), 4),
                      "kernel_frac_min": min(r["kernel_frac"] for r in sel),
                      "kernel_frac_max": max(r["kernel_frac"] for r in sel)}
    top = max(classes, key=lambda c: classes[c]["kernel_s"])
    sel = [r for r in rows if r["class"] == top]
    tk = sum(r["kernel_us"] for r in sel) / 1e6
    if top == "hbm":
        ach = sum(r["alg_bytes"] for r in sel) / tk / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        ach = sum(r["alg_flops"] for r in sel) / tk / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof.update({"frac": round(ach / roof["peak"], 4), "traffic": None,
                 "kernel": f"attn_mixed_kernel<{d}, {'true' if args.window > 0 else 'false'}> "
                           "(the sweep's steps of this class)"})
    tok = sum(r["query_tokens"] for r in rows)
    span = sum(r["span_us"] for r in rows) / 1e6
    log(f"[bench] sweep: {len(rows)} steps, {tok} query tokens, device {span * 1e3:.2f} ms; "
        + ", ".join(f"{c}: {v['steps']} steps {v['kernel_frac_of_peak']:.3f} of peak" for c, v in classes.items()))
    rec = {
        "metric": METRIC, "value": round(tok / span, 1), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(span / len(rows) * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V; no dataset)",
        "config": {"workload": w.name.replace("512@19456", "every512") + "_sweep", "steps_swept": len(rows),
                   "q_heads": hq, "kv_heads": hkv, "head_dim": d, "page_size": 16,
                   "sliding_window": args.window,
                   "timing": f"each step --steps times after --warmup untimed runs, enqueued back to back from "
                             f"the same builder state; steps under 1 GB cold (--cold {args.cold}, 1 GiB {args.flush} before "
                             f"each run); per step the median device span (append .. combine) and kernel time"},
        "roofline": roof,
        "sweep": {"classes": classes, "per_step": rows},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def kernel_clock_mhz(burst, lib, dev, n=5):
    """Shader clock (MHz) of the main attention kernel while it runs back to
    back: the library's clock hook (cb_profile_clock) has workgroup 0 record
    the shader-clock counter and the 100 MHz real-time counter at its start
    and end; ``burst()`` enqueues several calls, and the last call's record of
    each of ``n`` bursts is read."""
    import numpy as np
    import torch
    buf = torch.zeros(4, dtype=torch.int64, device=dev)
    vals = []
    lib.cb_profile_clock(buf.data_ptr())
    try:
        for _ in range(n):
            burst()
            torch.cuda.synchronize()
            c0, t0, c1, t1 = (int(x) for x in buf.cpu().tolist())
            if t1 > t0 and c1 > c0:
                vals.append((c1 - c0) * 100.0 / (t1 - t0))
    finally:
        lib.cb_profile_clock(None)
    if not vals:
        return None
    return {"mean": round(float(np.mean(vals)), 1), "min": round(float(np.min(vals)), 1),
            "max": round(float(np.max(vals)), 1), "samples": len(vals),
            "source": "s_memtime over s_memrealtime across workgroup 0 of the last of 8 back-to-back calls"}


def achievable_read_gbs(nbytes):
    """GB/s of the streaming-read probe (a child process) over ``nbytes``, or None."""
    probe = os.path.join(ROOT, "chunked_prefill_attention_amd", "hbm_probe")
    if not os.path.exists(probe):
        return None
    nbytes = (int(nbytes) + (1 << 20) - 1) >> 20 << 20
    try:
        r = subprocess.run([probe, "read", str(nbytes), "10"], capture_output=True, text=True, timeout=120)
        return float(json.loads(r.stdout.strip().splitlines()[-1])["GBps"]) if r.returncode == 0 else None
    except (subprocess.SubprocessError, ValueError, KeyError, IndexError):
        return None


def achievable_gemm_tflops(dev, n=16384, reps=5):
    """TFLOP/s of a plain bf16 GEMM (n x n x n, the vendor BLAS behind torch.matmul,
    contiguous operands) on this GPU: the dense-matrix rate the chip sustains
    in practice (the largest of 4096..16384 cubes measured best), for comparison
    with MFMA-bound kernels.  None on failure."""
    import torch
    try:
        a = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
        b = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
        c = a @ b
        torch.cuda.synchronize()
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        del a, b, c
        return round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    except Exception:  # pragma: no cover
        return None


def cpu_baseline(desc, q, hist, hq, hkv, d, budget_s, gpu_out, window=0):
    """Time the fp64 oracle on the step's sequences (test infrastructure)."""
    import numpy as np
    from oracle import attention as ora
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] + [1])
        blas_name = blas[0].get("internal_api", "?") if blas else "none"
    except Exception:  # pragma: no cover
        threads, blas_name = 1, "?"
    import workloads as wl
    scale = wl.softmax_scale(d)
    qh = q.float().cpu().numpy()
    gh = gpu_out.float().cpu().numpy()
    seqs = []
    for s in range(desc.num_seqs):
        i = int(desc.req_ids[s])
        c = int(desc.context_lens[s])
        a, e = int(desc.query_start_loc[s]), int(desc.query_start_loc[s + 1])
        seqs.append((qh[a:e], hist[i][0][:c].float().cpu().numpy(), hist[i][1][:c].float().cpu().numpy(), a, e))
    tokens, t_used, reps, worst = 0, 0.0, 0, 0.0
    while True:
        t0 = time.perf_counter()
        for qq, kk, vv, a, e in seqs:
            ref = ora.attend(qq, kk, vv, scale, window=window)
            if reps == 0:
                worst = max(worst, float(np.abs(ref - gh[a:e]).max()))
        t_used += time.perf_counter() - t0
        tokens += desc.num_tokens
        reps += 1
        if t_used >= budget_s or reps >= 50:
            break
    log(f"[bench] cpu oracle: {reps} x whole step in {t_used:.1f}s ({threads} BLAS threads, {blas_name}); "
        f"max |gpu - oracle| {worst:.3e}")
    return {"value": round(tokens / t_used, 1), "unit": "query tokens/s", "cores": len(os.sched_getaffinity(0)),
            "blas_threads": threads, "blas": blas_name, "kind": "oracle",
            "sample": f"the whole step ({desc.num_tokens} query tokens, {desc.num_seqs} sequences), "
                      f"{reps} repetition(s), fp64 numpy, {blas_name} BLAS",
            "max_abs_err_vs_gpu": worst}


if __name__ == "__main__":
    main()
