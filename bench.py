"""Benchmark: Gemma-4 12B-shaped attention over a device-resident KV cache.

One step = one pass of the layer stack: the 48 per-layer g4attn_decode calls
of the 12B-shaped decode stack (B = 16, context U{1024..4096}), captured once
into a HIP graph and replayed.  `value` is the KV bytes the step must read
(visible keys x KV heads x head_dim x 2 bytes, K and V, V counted once more
only on layers that have a V plane) divided by the step time, in GB/s.

Also reported on the same line:
  roofline      the dominant kernel (sliding-layer decode, head_dim 256),
                timed over a graph of the 40 sliding-layer launches;
  decode_step_with_append  the same step including the current token's
                K/V write: append + decode per layer vs the fused call;
  tp2_rank_decode  one tensor-parallel rank (TP=2) of the same decode stack;
  paged_decode  the same step through a paged cache (64-slot pages);
  long_context_decode  the long-context ragged stack (B = 64, context
                U{1..32768}, layers 20-47 KV-shared);
  softcap_decode  the 12B decode step with an attention-logit cap on every
                layer;
  small_decode  the launch-bound tiny 2-layer and E4B-shaped 12-layer stacks;
  prefill       the 12B-shaped 64-token prefill chunk stack (B = 4) after
                0, 960 and 4032 cached tokens, in TFLOP/s of visible-pair work
                (prefix 0 is launch-bound: read its us per step);
  cpu_baseline  the fp64 oracle on a bounded sample of the same decode
                workload, on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-prefill] [--copy-calib] [--main-only] [--long-context-only]
                       [--read-probe] [--gemm-probe] [--delivery-probe]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode-attn KV-read GB/s (% HBM peak) + prefill TFLOP/s, 12B shape, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes(wl, layer):
    """Algorithmic KV bytes one decode call of `layer` reads."""
    d = wl.layers[layer]
    keys = 0
    for L in wl.seq_lens:
        keys += min(L, d.window) if d.window > 0 else L
    return keys * d.n_kv_heads * d.head_dim * 2 * (1 if d.k_eq_v else 2)


DOMINANT_KERNEL = "attend_kernel<256, false, 4, false, false, false, true, false>"
PREFILL_KERNEL = "attend_kernel<512, true, 8, true, false, false, false, false>"
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "attend_12b_hbm_bytes.md")
KERNEL_SOURCE = os.path.join(ROOT, "decode_attention_gemma_amd", "csrc", "kernels.hip")
PLAN_SOURCE = os.path.join(ROOT, "decode_attention_gemma_amd", "csrc", "plan.cpp")


def source_hashes():
    """sha256[:16] of the kernel source and of the host plan (split planning
    and launch shapes), the two files a kernel's counters depend on."""
    import hashlib

    return {os.path.basename(f): hashlib.sha256(open(f, "rb").read()).hexdigest()[:16]
            for f in (KERNEL_SOURCE, PLAN_SOURCE)}


def counter_traffic(kernel: str):
    """HBM bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE)
    from the committed rocprofv3 summary, or None when that summary was taken
    on a different kernel source or host plan than the one built now."""
    try:
        text = open(COUNTER_SUMMARY).read()
        hashes = source_hashes()
    except OSError:
        return None
    if any(f"{name} sha256[:16]: {h}" not in text for name, h in hashes.items()):
        return None
    for row in text.splitlines():
        cells = [c.strip() for c in row.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0] == kernel:
            return int(round((float(cells[3]) + float(cells[5])) * 1e6))
    return None


def prefill_kv_bytes(wl, layer):
    """Unique K and V bytes a prefill call of `layer` reads: every key some
    token of the chunk sees, once (V only where the layer has a V plane)."""
    d = wl.layers[layer]
    keys = 0
    for s in wl.start_pos:
        lo = max(0, s - d.window + 1) if d.window > 0 else 0
        keys += s + wl.n_tok - lo
    return keys * d.n_kv_heads * d.head_dim * 2 * (1 if d.k_eq_v else 2)


def prefill_flops(wl, layer):
    """Visible (query, key) pairs x 4 x head_dim, over all query heads."""
    d = wl.layers[layer]
    pairs = 0
    for s in wl.start_pos:
        for t in range(wl.n_tok):
            p = s + t
            lo = max(0, p - d.window + 1) if d.window > 0 else 0
            pairs += p + 1 - lo
    return pairs * d.n_q_heads * 4 * d.head_dim


def graph_of(fn, stream):
    import torch

    with torch.cuda.stream(stream):
        fn()  # warm-up launch on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


def time_graph(g, warmup, reps, stats=None):
    """Median ms per replay over `reps` timed replays.  Replays run on the
    current stream, where a HIP event is recorded between consecutive
    replays; the timed region is bracketed by device synchronizations.  When
    `stats` is a dict it also receives the mean over the whole region."""
    import statistics

    import torch

    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(cur)
    for i in range(reps):
        g.replay()
        ev[i + 1].record(cur)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    if stats is not None:
        stats["mean_ms"] = ev[0].elapsed_time(ev[reps]) / reps
        stats["reps"] = reps
    return statistics.median(per)


def bench_decode(args, stream):
    import torch

    from decode_attention_gemma_amd import harness as H, workloads as W

    wl = W.g12b_decode()
    log(f"[bench] setup {wl.name}")
    st = H.make_stack(wl, "cuda")
    H.fill_cache(st, wl, "cuda")
    bufs = H.StepBuffers(wl, "cuda")
    step_graph = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream), stream)
    log(f"[bench] decode step: {args.warmup} warm-up, {args.steps} timed replays")
    t0 = time.perf_counter()
    stats = {}
    ms = time_graph(step_graph, args.warmup, args.steps, stats)
    wall = time.perf_counter() - t0
    step_bytes = sum(kv_bytes(wl, i) for i in range(wl.n_layers))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] decode step {ms*1e3:.1f} us, {gbs:.0f} GB/s (wall incl. warm-up {wall:.2f} s)")

    # dominant kernel: the sliding-layer decode (head_dim 256), one launch per
    # sliding layer so every launch streams a different cache region
    sliding = [i for i in range(wl.n_layers) if wl.layers[i].window > 0]
    dom_graph = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream, layers=sliding),
                         stream)
    dom_ms = time_graph(dom_graph, 3, max(args.steps, 20)) / len(sliding)
    dom_bytes = kv_bytes(wl, sliding[0])
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    log(f"[bench] sliding decode kernel {dom_ms*1e3:.1f} us/launch, {dom_gbs:.0f} GB/s")
    glob = [i for i in range(wl.n_layers) if wl.layers[i].window == 0]
    glob_graph = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream, layers=glob),
                          stream)
    glob_ms = time_graph(glob_graph, 3, max(args.steps, 20)) / len(glob)
    glob_gbs = kv_bytes(wl, glob[0]) / (glob_ms * 1e-3) / 1e9
    log(f"[bench] global decode kernel {glob_ms*1e3:.1f} us/launch, {glob_gbs:.0f} GB/s")
    out = {
        "wl": wl, "st": st, "bufs": bufs, "ms": ms, "mean_ms": stats["mean_ms"],
        "step_bytes": step_bytes, "gbs": gbs,
        "dom": {"ms": dom_ms, "bytes": dom_bytes, "gbs": dom_gbs},
        "glob": {"ms": glob_ms, "bytes": kv_bytes(wl, glob[0]), "gbs": glob_gbs},
    }
    return out


def bench_fused_step(args, stream):
    """The 12B decode step including the current token's K/V write, as a
    separate g4attn_append_kv + g4attn_decode per layer and as one fused
    g4attn_decode_append per layer."""
    import torch

    from decode_attention_gemma_amd import harness as H, workloads as W

    wl = W.g12b_decode()
    log(f"[bench] setup {wl.name} (with the token append)")
    st = H.make_stack(wl, "cuda")
    H.fill_cache(st, wl, "cuda")
    bufs = H.StepBuffers(wl, "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    knew, vnew = [], []
    for d in wl.layers:
        shape = (wl.batch, d.n_kv_heads, d.head_dim)
        knew.append(torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16))
        vnew.append(None if d.k_eq_v else
                    torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16))
    pos = (bufs.lens - 1).to(torch.int32)
    sid = stream.cuda_stream

    def separate():
        for i in range(wl.n_layers):
            st.append_kv(i, knew[i][:, None], None if vnew[i] is None else vnew[i][:, None], pos,
                         max_end_pos=bufs.max_len, stream=sid)
            st.decode(i, bufs.q[i], bufs.lens, bufs.max_len, bufs.out[i], sid)

    def fused():
        for i in range(wl.n_layers):
            st.decode_append(i, bufs.q[i], knew[i], vnew[i], bufs.lens, bufs.max_len, bufs.out[i],
                             sid)

    ms_sep = time_graph(graph_of(separate, stream), args.warmup, args.steps)
    ms_fus = time_graph(graph_of(fused, stream), args.warmup, args.steps)
    log(f"[bench] decode step with token append: separate {ms_sep*1e3:.1f} us, "
        f"fused {ms_fus*1e3:.1f} us")
    del st, bufs
    torch.cuda.empty_cache()
    return {"separate_append_then_decode_us": round(ms_sep * 1e3, 2),
            "fused_decode_append_us": round(ms_fus * 1e3, 2)}


def bench_rank_decode(args, stream):
    """One tensor-parallel rank (TP=2) of the 12B decode stack, whole step."""
    import torch

    from decode_attention_gemma_amd import harness as H, workloads as W

    wl = W.g12b_tp2_rank_decode()
    log(f"[bench] setup {wl.name}")
    st = H.make_stack(wl, "cuda")
    H.fill_cache(st, wl, "cuda")
    bufs = H.StepBuffers(wl, "cuda")
    g = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream), stream)
    ms = time_graph(g, args.warmup, args.steps)
    step_bytes = sum(kv_bytes(wl, i) for i in range(wl.n_layers))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] TP=2 rank decode step {ms*1e3:.1f} us, {gbs:.0f} GB/s")
    del st, bufs, g
    torch.cuda.empty_cache()
    return {"workload": wl.name + " (sliding 8q/4kv, global 8q/1kv replicated)",
            "us_per_step": round(ms * 1e3, 2), "kv_bytes_per_step": step_bytes,
            "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_long_decode(args, stream):
    """The long-context ragged decode stack: 12B geometry with layers 20-47
    reading earlier owners' caches, B = 64, context U{1..32768}, 1% outliers."""
    import torch

    from decode_attention_gemma_amd import harness as H, workloads as W

    wl = W.long_decode()
    log(f"[bench] setup {wl.name}")
    st = H.make_stack(wl, "cuda")
    H.fill_cache(st, wl, "cuda")
    bufs = H.StepBuffers(wl, "cuda")
    g = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream), stream)
    ms = time_graph(g, args.warmup, args.steps)
    step_bytes = sum(kv_bytes(wl, i) for i in range(wl.n_layers))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] long-context decode step {ms*1e3:.1f} us, {gbs:.0f} GB/s")
    del st, bufs, g
    torch.cuda.empty_cache()
    return {"workload": wl.name + " (12B geometry, layers 20-47 KV-shared), B=64, "
                                  "context U{1..32768}",
            "us_per_step": round(ms * 1e3, 2), "kv_bytes_per_step": step_bytes,
            "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_small_decode(args, stream):
    """The launch-bound decode stacks: the tiny 2-layer stack and the E4B-shaped
    12-layer stack with KV sharing (B = 1, context 511), in us per step."""
    import torch

    from decode_attention_gemma_amd import harness as H, workloads as W

    out = {}
    for key, mk in (("tiny_2layer", W.tiny_stack), ("e4b_12layer", W.e4b_decode)):
        wl = mk()
        log(f"[bench] setup {wl.name}")
        st = H.make_stack(wl, "cuda")
        H.fill_cache(st, wl, "cuda")
        bufs = H.StepBuffers(wl, "cuda")
        g = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream), stream)
        ms = time_graph(g, args.warmup, max(args.steps, 50))
        step_bytes = sum(kv_bytes(wl, i) for i in range(wl.n_layers))
        log(f"[bench] {wl.name}: {ms*1e3:.1f} us/step, {step_bytes/ms/1e6:.0f} GB/s")
        out[key] = {"workload": wl.name, "us_per_step": round(ms * 1e3, 2),
                    "us_per_layer": round(ms * 1e3 / wl.n_layers, 2),
                    "kv_bytes_per_step": step_bytes,
                    "gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1)}
        del st, bufs, g
        torch.cuda.empty_cache()
    return out


def bench_softcap_decode(args, stream):
    """The 12B decode stack with an attention-logit cap of 50 on every layer."""
    import dataclasses

    import torch

    from decode_attention_gemma_amd import harness as H, workloads as W

    wl = W.g12b_decode()
    wl.layers = [dataclasses.replace(d, softcap=50.0) for d in wl.layers]
    log(f"[bench] setup {wl.name} (logit cap 50)")
    st = H.make_stack(wl, "cuda")
    H.fill_cache(st, wl, "cuda")
    bufs = H.StepBuffers(wl, "cuda")
    g = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream), stream)
    ms = time_graph(g, args.warmup, args.steps)
    step_bytes = sum(kv_bytes(wl, i) for i in range(wl.n_layers))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] softcap decode step {ms*1e3:.1f} us, {gbs:.0f} GB/s")
    del st, bufs, g
    torch.cuda.empty_cache()
    return {"workload": wl.name + ", every layer capped at c = 50",
            "us_per_step": round(ms * 1e3, 2), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_paged_decode(args, stream):
    """The 12B decode step through a paged cache: pages of `--page-size`
    slots (64 by default) in a seeded random order over a pool of arbitrary
    bits, one block table for all layers."""
    import torch

    from decode_attention_gemma_amd import harness as H, workloads as W

    wl = W.g12b_decode()
    page = args.page_size
    log(f"[bench] setup {wl.name} (paged cache, {page}-slot pages)")
    st = H.make_paged_stack(wl, page_size=page, device="cuda")
    H.fill_cache(st, wl, "cuda")
    bufs = H.StepBuffers(wl, "cuda")
    g = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream), stream)
    ms = time_graph(g, args.warmup, args.steps)
    step_bytes = sum(kv_bytes(wl, i) for i in range(wl.n_layers))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    # the same step with each token's K/V write fused into its decode launch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    knew, vnew = [], []
    for d in wl.layers:
        shape = (wl.batch, d.n_kv_heads, d.head_dim)
        knew.append(torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16))
        vnew.append(None if d.k_eq_v else
                    torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16))
    sid = stream.cuda_stream

    def fused():
        for i in range(wl.n_layers):
            st.decode_append(i, bufs.q[i], knew[i], vnew[i], bufs.lens, bufs.max_len, bufs.out[i],
                             sid)

    ms_fus = time_graph(graph_of(fused, stream), args.warmup, args.steps)
    log(f"[bench] paged decode step {ms*1e3:.1f} us, {gbs:.0f} GB/s; "
        f"with the fused token append {ms_fus*1e3:.1f} us")
    del st, bufs, g
    torch.cuda.empty_cache()
    return {"workload": wl.name + f", paged ({page}-slot pages, permuted)",
            "us_per_step": round(ms * 1e3, 2), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "fused_decode_append_us": round(ms_fus * 1e3, 2)}


def bench_prefill(prefix, args, stream):
    import torch

    from decode_attention_gemma_amd import harness as H, workloads as W

    wl = W.g12b_prefill(prefix)
    log(f"[bench] setup {wl.name}")
    st = H.make_stack(wl, "cuda")
    H.fill_cache(st, wl, "cuda")
    bufs = H.StepBuffers(wl, "cuda")
    g = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream), stream)
    ms = time_graph(g, args.warmup, args.steps)
    flops = sum(prefill_flops(wl, i) for i in range(wl.n_layers))
    tf = flops / (ms * 1e-3) / 1e12
    glob = [i for i in range(wl.n_layers) if wl.layers[i].window == 0]
    slid = [i for i in range(wl.n_layers) if wl.layers[i].window > 0]
    gg = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream, layers=glob), stream)
    gms = time_graph(gg, 2, max(args.steps, 20)) / len(glob)
    sg = graph_of(lambda: H.run_step(st, bufs, stream=stream.cuda_stream, layers=slid), stream)
    sms = time_graph(sg, 2, max(args.steps, 20)) / len(slid)
    gtf = prefill_flops(wl, glob[0]) / (gms * 1e-3) / 1e12
    stf = prefill_flops(wl, slid[0]) / (sms * 1e-3) / 1e12
    sgbs = prefill_kv_bytes(wl, slid[0]) / (sms * 1e-3) / 1e9
    log(f"[bench] prefill P={prefix}: {ms*1e3:.1f} us/step, {tf:.1f} TFLOP/s; "
        f"global layer {gms*1e3:.1f} us, {gtf:.1f} TFLOP/s; sliding layer {sms*1e3:.1f} us, "
        f"{stf:.1f} TFLOP/s, {sgbs:.0f} GB/s of unique KV")
    del st, bufs, g, gg, sg
    torch.cuda.empty_cache()
    return {"us_per_step": round(ms * 1e3, 2), "tflops": round(tf, 2),
            "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4), "gflop_per_step": round(flops / 1e9, 2),
            "global_layer_us": round(gms * 1e3, 2), "global_layer_tflops": round(gtf, 2),
            "global_layer_gflop": round(prefill_flops(wl, glob[0]) / 1e9, 3),
            "sliding_layer_us": round(sms * 1e3, 2), "sliding_layer_tflops": round(stf, 2),
            "sliding_layer_kv_gbs": round(sgbs, 1)}


CPU_REPS = 4  # oracle passes over the decode step: about 5 s of compute on 16 cores


def _host64(t):
    import torch

    return t.to("cpu", torch.float64).numpy()


def probe_lib():
    """libg4probe.so (the hardware-rate probes), built beside the library."""
    import ctypes

    from decode_attention_gemma_amd import build as B

    if not os.path.exists(B.PROBE_LIB):
        raise ImportError(f"{B.PROBE_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.g4probe_read.restype = ctypes.c_int
    lib.g4probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.g4probe_mfma.restype = ctypes.c_int
    lib.g4probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.g4probe_lds.restype = ctypes.c_int
    lib.g4probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_void_p]
    lib.g4probe_l2.restype = ctypes.c_int
    lib.g4probe_l2.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def _median_launch_ms(stream, launch, reps):
    """Median of `reps` HIP-event timings of launch() on `stream`, after one
    untimed launch."""
    import torch

    times = []
    for it in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = launch()
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"probe launch: hip error {rc}")
        e1.synchronize()
        if it > 0:
            times.append(e0.elapsed_time(e1))
    times.sort()
    return times[len(times) // 2]


def delivery_probe(args, stream):
    """Per-CU operand delivery, the bounds of the prefill kernels
    (libg4probe.so): the LDS read rate of 16-byte and of transposing 8-byte
    reads, and the L2 -> CU load rate into registers or straight into LDS,
    with 4, 8 and 16 waves per CU (one workgroup on each of the 256 CUs).
    Bytes per clock at the 2.4 GHz peak engine clock."""
    import ctypes

    import torch

    lib = probe_lib()
    sink = torch.zeros(1 << 14, dtype=torch.uint8, device="cuda")
    cs = ctypes.c_void_p(stream.cuda_stream)
    reps = max(args.steps, 10)
    res = {}
    n_cu, clk = 256, 2.4e9
    with torch.cuda.stream(stream):
        for tr in (0, 1):
            for threads in (256, 512, 1024):
                iters = 2048
                ms = _median_launch_ms(stream, lambda: lib.g4probe_lds(
                    tr, n_cu, threads, iters, sink.data_ptr(), cs), reps)
                per_cu = (threads // 64) * iters * 4096 / (ms * 1e-3)
                key = f"lds_{'tr_b64' if tr else 'b128'}_{threads // 64}w"
                res[key] = round(per_cu / clk, 1)
                log(f"[bench] lds probe {'ds_read_b64_tr_b16' if tr else 'ds_read_b128'}, "
                    f"{threads // 64} waves per CU: {ms*1e3:.0f} us, {per_cu/1e9:.0f} GB/s per CU, "
                    f"{per_cu/clk:.0f} B/clk")
        for region in (256 << 10, 1 << 20):
            buf = torch.zeros(8 * region, dtype=torch.uint8, device="cuda")
            passes = (64 << 20) // region
            for to_lds in (0, 1):
                for threads in (256, 512, 1024):
                    ms = _median_launch_ms(stream, lambda: lib.g4probe_l2(
                        to_lds, buf.data_ptr(), region, n_cu, threads, passes, sink.data_ptr(),
                        cs), reps)
                    per_cu = region * passes / (ms * 1e-3)
                    key = f"l2_{region >> 10}KiB_{'lds' if to_lds else 'vgpr'}_{threads // 64}w"
                    res[key] = round(per_cu / 1e9, 1)
                    log(f"[bench] l2 probe {region >> 10} KiB per XCD, "
                        f"{'into LDS' if to_lds else 'into registers'}, {threads // 64} waves per "
                        f"CU: {ms*1e3:.0f} us, {per_cu/1e9:.0f} GB/s per CU ({per_cu/clk:.0f} "
                        f"B/clk), {n_cu * per_cu / 1e12:.1f} TB/s in all")
            del buf
    del sink
    torch.cuda.empty_cache()
    return res


def read_probe(args, stream):
    """HBM streaming read rate (the practical bound for the decode kernels):
    one read kernel (libg4probe.so, built beside the library) over 134 MB
    regions, the sliding decode layer's bytes, each launch a different region
    of a 4 GiB buffer so that nothing is left in the 256 MB MALL from the
    previous launch, and over the whole buffer at once; plain and
    non-temporal loads, several grid sizes; medians of HIP-event timings."""
    import ctypes

    import torch

    lib = probe_lib()
    region = 134217728
    total = 4 << 30
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    buf.view(torch.int32).fill_(0x3c003c00)
    sink = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    n_regions = total // region
    res = {}
    with torch.cuda.stream(stream):
        for nt in (0, 1):
            for n_wg in (256, 512, 1024, 2048):
                times = []
                for it in range(max(args.steps, 20) + 3):
                    off = (it % n_regions) * region
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    rc = lib.g4probe_read(buf.data_ptr() + off, region, nt, n_wg, sink.data_ptr(),
                                          ctypes.c_void_p(stream.cuda_stream))
                    e1.record(stream)
                    if rc != 0:
                        raise RuntimeError(f"g4probe_read: hip error {rc}")
                    e1.synchronize()
                    if it >= 3:
                        times.append(e0.elapsed_time(e1))
                times.sort()
                ms = times[len(times) // 2]
                key = f"{'nt' if nt else 'plain'}_134MB_{n_wg}wg"
                res[key] = round(region / (ms * 1e-3) / 1e9, 1)
                log(f"[bench] read probe 134 MB regions, {'non-temporal' if nt else 'plain'} loads, "
                    f"{n_wg} workgroups: {ms*1e3:.1f} us, {res[key]:.0f} GB/s")
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            times = []
            for it in range(6):
                e0.record(stream)
                lib.g4probe_read(buf.data_ptr(), total, nt, 2048, sink.data_ptr(),
                                 ctypes.c_void_p(stream.cuda_stream))
                e1.record(stream)
                e1.synchronize()
                if it >= 1:
                    times.append(e0.elapsed_time(e1))
            times.sort()
            ms = times[len(times) // 2]
            key = f"{'nt' if nt else 'plain'}_4GiB_2048wg"
            res[key] = round(total / (ms * 1e-3) / 1e9, 1)
            log(f"[bench] read probe 4 GiB at once, {'non-temporal' if nt else 'plain'} loads: "
                f"{ms*1e3:.0f} us, {res[key]:.0f} GB/s")
    del buf, sink
    torch.cuda.empty_cache()
    return res


def gemm_probe(args, stream):
    """Achievable dense bf16 matrix-core rates, against the 2.5 PFLOP/s spec
    figure: the issue rate of back-to-back 16x16x32 bf16 MFMAs with no memory
    traffic (libg4probe.so, 256 workgroups, one or two waves per SIMD, 4 or 8
    independent chains per wave), and large square bf16 GEMMs through
    torch.matmul (the vendor BLAS, contiguous 2-D operands, fp32
    accumulate).  Medians of HIP-event timings."""
    import ctypes

    import torch

    lib = probe_lib()
    res = {}
    sink = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    iters = 4096
    with torch.cuda.stream(stream):
        for threads in (256, 512):
            for chains in (4, 8):
                times = []
                for it in range(8):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    rc = lib.g4probe_mfma(256, threads, chains, iters, sink.data_ptr(),
                                          ctypes.c_void_p(stream.cuda_stream))
                    e1.record(stream)
                    if rc != 0:
                        raise RuntimeError(f"g4probe_mfma: hip error {rc}")
                    e1.synchronize()
                    if it >= 2:
                        times.append(e0.elapsed_time(e1))
                times.sort()
                ms = times[len(times) // 2]
                flops = 256 * (threads // 64) * iters * chains * 16 * 16 * 32 * 2
                tf = flops / (ms * 1e-3) / 1e12
                res[f"mfma_issue_{threads // 256}wps_{chains}ch"] = round(tf, 1)
                log(f"[bench] mfma probe {threads // 256} wave(s) per SIMD, {chains} chains: "
                    f"{ms*1e3:.0f} us, {tf:.0f} TFLOP/s ({tf / BF16_PEAK_TFLOPS:.1%} of spec)")
        for n in (8192, 16384):
            g = torch.Generator(device="cuda").manual_seed(7)
            a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
            b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
            c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
            times = []
            for it in range(max(args.steps, 20) + 3):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                torch.matmul(a, b, out=c)
                e1.record(stream)
                e1.synchronize()
                if it >= 3:
                    times.append(e0.elapsed_time(e1))
            times.sort()
            ms = times[len(times) // 2]
            tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
            res[f"bf16_gemm_{n}"] = round(tf, 1)
            log(f"[bench] gemm probe {n}x{n}x{n} bf16: {ms*1e3:.0f} us, {tf:.0f} TFLOP/s "
                f"({tf / BF16_PEAK_TFLOPS:.1%} of the {BF16_PEAK_TFLOPS:.0f} TFLOP/s spec)")
            del a, b, c
    torch.cuda.empty_cache()
    return res


def cpu_baseline(dec, gpu_prefill_tflops=None, gpu_long_gbs=None):
    """The fp64 oracle, timed on the host cores on bounded samples of the
    benchmarked workloads (inputs are the same seeded bf16 tensors, copied to
    the host and widened to fp64 outside the timed regions):
      decode   every layer and sequence of the 12B decode step, CPU_REPS passes;
      prefill  the 64-token chunk at prefix 4032: its first 12 layers (10
               sliding, 2 global) for all 4 sequences (flops counted as the
               metric's visible pairs);
      long     the long-context ragged stack: one sliding and one global owner
               layer for all 64 sequences."""
    import numpy as np  # noqa: F401
    import torch

    from decode_attention_gemma_amd import workloads as W
    from oracle import attn64 as O

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    wl, bufs = dec["wl"], dec["bufs"]
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    log(f"[bench] cpu baseline: fp64 oracle, all {wl.n_layers} layers x {wl.batch} sequences, "
        f"{CPU_REPS} passes")
    dt = 0.0
    nbytes = 0
    for layer in range(wl.n_layers):
        d = wl.layers[layer]
        o = wl.owner(layer)
        q = _host64(bufs.q[layer])
        inputs = []
        for b in range(wl.batch):
            pos0, _ = W.kv_span(wl, o, b)
            K = _host64(W.kv_rows(wl, o, b, "k", "cuda"))
            V = None if d.k_eq_v else _host64(W.kv_rows(wl, o, b, "v", "cuda"))
            inputs.append((q[b], K, V, wl.seq_lens[b], pos0))
            L = wl.seq_lens[b]
            keys = min(L, d.window) if d.window > 0 else L
            nbytes += CPU_REPS * keys * d.n_kv_heads * d.head_dim * 2 * (1 if d.k_eq_v else 2)
        t0 = time.perf_counter()
        for _ in range(CPU_REPS):
            for qb, K, V, L, pos0 in inputs:
                O.decode_sequence(d, qb, K, V, L, k_pos0=pos0)
        dt += time.perf_counter() - t0
        del inputs
    gbs = nbytes / dt / 1e9
    log(f"[bench] cpu baseline decode {dt:.2f} s for {nbytes/1e9:.3f} GB -> {gbs:.3f} GB/s")

    # prefill chunk, prefix 4032: the first 12 layers (10 sliding, 2 global),
    # all 4 sequences
    pw = W.g12b_prefill(4032)
    p_dt, p_flops = 0.0, 0
    for layer in range(12):
        d = pw.layers[layer]
        q = _host64(W.q_tensor(pw, layer, "cuda"))
        for b in range(pw.batch):
            pos0, _ = W.kv_span(pw, layer, b)
            K = _host64(W.kv_rows(pw, layer, b, "k", "cuda"))
            V = None if d.k_eq_v else _host64(W.kv_rows(pw, layer, b, "v", "cuda"))
            t0 = time.perf_counter()
            O.prefill_sequence(d, q[b], K, V, pw.start_pos[b], k_pos0=pos0)
            p_dt += time.perf_counter() - t0
        p_flops += prefill_flops(pw, layer)
    p_gfs = p_flops / p_dt / 1e9
    log(f"[bench] cpu baseline prefill {p_dt:.2f} s for {p_flops/1e9:.2f} GFLOP -> "
        f"{p_gfs:.3f} GFLOP/s")

    # long-context ragged decode: one sliding and one global owner layer, all
    # 64 sequences
    lw = W.long_decode()
    l_dt, l_bytes = 0.0, 0
    for layer in (0, 5):
        d = lw.layers[layer]
        q = _host64(W.q_tensor(lw, layer, "cuda"))
        for b in range(lw.batch):
            pos0, _ = W.kv_span(lw, layer, b)
            K = _host64(W.kv_rows(lw, layer, b, "k", "cuda"))
            V = None if d.k_eq_v else _host64(W.kv_rows(lw, layer, b, "v", "cuda"))
            t0 = time.perf_counter()
            O.decode_sequence(d, q[b], K, V, lw.seq_lens[b], k_pos0=pos0)
            l_dt += time.perf_counter() - t0
            L = lw.seq_lens[b]
            keys = min(L, d.window) if d.window > 0 else L
            l_bytes += keys * d.n_kv_heads * d.head_dim * 2 * (1 if d.k_eq_v else 2)
            del K, V
    l_gbs = l_bytes / l_dt / 1e9
    log(f"[bench] cpu baseline long-context decode {l_dt:.2f} s for {l_bytes/1e9:.3f} GB -> "
        f"{l_gbs:.3f} GB/s")
    if ctx is not None:
        ctx.restore_original_limits()
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_step": round(dt / CPU_REPS * 1e6, 1),
            "sample": f"{CPU_REPS} passes over one full step of the same decode workload (48 "
                      f"layers x 16 sequences, {nbytes/CPU_REPS/1e9:.2f} GB of bf16 KV per "
                      f"pass), fp64 numpy oracle, compute timed {dt:.1f} s, BLAS threads "
                      f"limited to the {cores} cores",
            "prefill": {"value": round(p_gfs, 3), "unit": "GFLOP/s", "kind": "oracle",
                        "seconds": round(p_dt, 2),
                        "gpu_over_oracle": (round(gpu_prefill_tflops * 1e3 / p_gfs, 1)
                                            if gpu_prefill_tflops else None),
                        "sample": "64-token prefill chunk at prefix 4032, layers 0-11 (10 "
                                  f"sliding, 2 global), all 4 sequences: {p_flops/1e9:.2f} "
                                  "GFLOP of visible-pair work"},
            "long_context": {"value": round(l_gbs, 3), "unit": "GB/s", "kind": "oracle",
                             "seconds": round(l_dt, 2),
                             "gpu_over_oracle": (round(gpu_long_gbs / l_gbs, 1)
                                                 if gpu_long_gbs else None),
                             "sample": "long-context ragged decode, layers 0 (sliding) and 5 "
                                       f"(global), all 64 sequences: {l_bytes/1e9:.3f} GB of "
                                       "KV"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one 1 GiB device copy, the reference for HBM byte counters")
    ap.add_argument("--long-context-only", action="store_true",
                    help="run only the long-context ragged decode stack and log its step time "
                         "(no JSON line; for per-kernel profiles of that workload)")
    ap.add_argument("--read-probe", action="store_true",
                    help="run only the HBM read-rate probe (plain and non-temporal loads) and "
                         "log its rates (no JSON line)")
    ap.add_argument("--delivery-probe", action="store_true",
                    help="run only the LDS and L2 -> CU delivery probes (the prefill kernels' "
                         "operand paths) and exit")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="run only the bf16 GEMM probe (the achievable matrix-core rate) and "
                         "log its rates (no JSON line)")
    ap.add_argument("--paged-only", action="store_true",
                    help="run only the 12B decode step, unpaged and through the paged cache, "
                         "and log both times (no JSON line; for the paged layout's profiles)")
    ap.add_argument("--page-size", type=int, default=64,
                    help="slots per page of the paged decode step (a multiple of 64)")
    ap.add_argument("--main-only", action="store_true",
                    help="skip the TP=2 rank stack, the fused-append step and the paged step, "
                         "which launch the decode kernels at other shapes or in other "
                         "instances (for per-kernel profiler averages)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention path here runs on a single "
              "MI355X (see DESIGN.md for how it would shard); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_attention_gemma_amd import g4attn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    g4attn.load()
    stream = torch.cuda.Stream()
    if args.long_context_only:
        bench_long_decode(args, stream)
        return
    if args.paged_only:
        bench_decode(args, stream)
        bench_paged_decode(args, stream)
        return
    if args.read_probe:
        read_probe(args, stream)
        return
    if args.gemm_probe:
        gemm_probe(args, stream)
        return
    if args.delivery_probe:
        delivery_probe(args, stream)
        return
    if args.copy_calib:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB device-to-device copy done")
        del src, dst
        torch.cuda.empty_cache()
    dec = bench_decode(args, stream)
    rank = None if args.main_only else bench_rank_decode(args, stream)
    fused = None if args.main_only else bench_fused_step(args, stream)
    paged = None if args.main_only else bench_paged_decode(args, stream)
    long_ctx = None if args.main_only else bench_long_decode(args, stream)
    capped = None if args.main_only else bench_softcap_decode(args, stream)
    small = None if args.main_only else bench_small_decode(args, stream)
    prefill = {}
    if not args.no_prefill:
        for p in ((960, 4032) if args.main_only else (0, 960, 4032)):
            prefill[f"prefix_{p}"] = bench_prefill(p, args, stream)
    p4032 = prefill.get("prefix_4032")
    cpu = None if args.no_cpu_baseline else cpu_baseline(
        dec, p4032["tflops"] if p4032 else None, long_ctx["gbs"] if long_ctx else None)
    prefill_line = None
    if p4032:
        prefill_line = {
            "metric": "prefill TFLOP/s (4 x head_dim flops per visible query-key pair)",
            "value": p4032["tflops"],
            "unit": "TFLOP/s",
            "frac": round(p4032["tflops"] / BF16_PEAK_TFLOPS, 4),
            "ms_per_step": round(p4032["us_per_step"] / 1e3, 4),
            "gflop_per_step": p4032["gflop_per_step"],
            "workload": "12B-shaped 48-layer 64-token prefill chunk (40 sliding W1024 16q/8kv "
                        "D256 + 8 global 16q/1kv D512 k_eq_v), B=4, prefix 4032",
            "roofline": {
                "kernel": PREFILL_KERNEL + " (global-layer prefill, prefix 4032)",
                "bound": "mfma",
                "achieved": p4032["global_layer_tflops"],
                "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(p4032["global_layer_tflops"] / BF16_PEAK_TFLOPS, 4),
                "us_per_launch": p4032["global_layer_us"],
                "gflop_per_launch": p4032["global_layer_gflop"],
            },
            "sliding_layer_us": p4032["sliding_layer_us"],
            "sliding_layer_kv_gbs": p4032["sliding_layer_kv_gbs"],
        }
        for k, v in prefill.items():
            prefill_line[f"{k}_us_per_step"] = v["us_per_step"]
            prefill_line[f"{k}_tflops"] = v["tflops"]

    wl = dec["wl"]
    dom = dec["dom"]
    line = {
        "metric": METRIC,
        "value": round(dec["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 4),
        "ms_per_step_mean": round(dec["mean_ms"], 4),
        "timing": "median of the timed replays (HIP events between replays)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, no weights)",
        "config": {
            "workload": "12B-shaped 48-layer decode stack (40 sliding W1024 16q/8kv D256 + "
                        "8 global 16q/1kv D512 k_eq_v), B=16, context U{1024..4096}",
            "batch": wl.batch, "layers": wl.n_layers, "seq_lens": wl.seq_lens,
            "kv_bytes_per_step": dec["step_bytes"],
            "hbm_frac": round(dec["gbs"] / HBM_PEAK_GBS, 4),
            "global_layer_decode_gbs": round(dec["glob"]["gbs"], 1),
        },
        "roofline": {
            "kernel": DOMINANT_KERNEL + " (sliding-layer decode)",
            "bound": "hbm",
            "achieved": round(dom["gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic(DOMINANT_KERNEL),
            "us_per_launch": round(dom["ms"] * 1e3, 2),
            "bytes_per_launch": dom["bytes"],
        },
        "decode_step_with_append": fused,
        "tp2_rank_decode": rank,
        "paged_decode": paged,
        "long_context_decode": long_ctx,
        "softcap_decode": capped,
        "small_decode": small,
        "prefill": prefill_line,
        "prefill_by_prefix": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
