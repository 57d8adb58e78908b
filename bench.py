"""Benchmark of the FP8 attention forward on one MI355X.

One step = one split-KV decode step over the paged GQA decode workload (64 sequences, 32 query
/ 8 KV heads, d = 128, one query token, 16-token pages, lengths uniform in [1024, 8192],
per-(batch, kv head) descales): the device-computed balanced split schedule, the decode pass and
the combine, captured in a HIP graph and replayed, as the pages time decode. The headline value
is the step's K+V bandwidth in GB/s. The causal-prefill workload (B = 2, 8192 x 8192, 32/8
heads, d = 128) is timed next to it and reported in TFLOP/s under "prefill".

Prints one JSON line. Inputs are resident in HBM before timing; the dominant kernel's own
average duration is measured with HIP events on its launch stream around a run of back-to-back
decode launches (and, per launch, around the decode kernel of every step of an eager loop).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np
import torch

from fa8_fwd_amd import binding
from fa8_fwd_amd import inputs as gen

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA


# ---------------------------------------------------------------------------------------------
# work counts (algorithmic: what the method must read/write/compute, not what a kernel wastes)
# ---------------------------------------------------------------------------------------------

def visible_pairs(inp) -> int:
    """(query, key) pairs visible under the causal/window mask, summed over batches."""
    sq, sk = inp.seqlens_q(), inp.seqlens_k()
    total = 0
    wr = 0 if inp.causal else inp.window_right
    for b in range(inp.batch):
        i = np.arange(int(sq[b]), dtype=np.int64)
        ip = i + int(sk[b]) - int(sq[b])
        hi = np.full_like(i, int(sk[b]))
        if wr >= 0:
            hi = np.minimum(hi, ip + wr + 1)
        lo = np.zeros_like(i)
        if inp.window_left >= 0:
            lo = np.maximum(lo, ip - inp.window_left)
        total += int(np.clip(hi - lo, 0, None).sum())
    return total


def prefill_flop(inp) -> int:
    """2 * (d + dv) FLOP per visible pair and query head (QK^T and PV)."""
    return visible_pairs(inp) * inp.heads_q * 2 * (inp.d + inp.dv)


def decode_kernel_bytes(inp) -> int:
    """Bytes the split-KV decode kernel must move: every visible K and V row once
    (sum_b s_b * Hkv * (d + dv)), the Q rows, the block-table entries and lengths, the descales."""
    sk = inp.seqlens_k()
    sq = inp.seqlens_q()
    kv = int(sk.sum()) * inp.heads_kv * (inp.d + inp.dv)
    q = int(sq.sum()) * inp.heads_q * inp.d
    table = int(((sk + inp.page_size - 1) // inp.page_size).sum()) * 4 if inp.block_table is not None else 0
    lens = inp.batch * 4 * 2
    desc = sum(0 if x is None else x.size * 4 for x in (inp.q_descale, inp.k_descale, inp.v_descale))
    return kv + q + table + lens + desc


def decode_step_bytes(inp) -> int:
    """Whole decode step: the kernel's bytes plus the bf16 output written once."""
    return decode_kernel_bytes(inp) + int(inp.seqlens_q().sum()) * inp.heads_q * inp.dv * 2


# ---------------------------------------------------------------------------------------------
# HBM traffic from hardware counters (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE), recorded in a
# committed summary under profiles/ together with the hash of the kernel sources it was taken on
# ---------------------------------------------------------------------------------------------

def kernel_source_hash() -> str:
    """sha256 over the library's device and host sources (what decides the launched kernels)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fa8_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def recorded_traffic(summary: str):
    """HBM bytes per launch recorded in profiles/<summary>, or None when there is no record or
    the sources have changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", summary)) as f:
            text = f.read()
    except OSError:
        return None
    sha = re.search(r"kernel source sha256: `([0-9a-f]{64})`", text)
    nbytes = re.search(r"traffic per launch: ([0-9]+) bytes", text)
    if not (sha and nbytes) or sha.group(1) != kernel_source_hash():
        return None
    return int(nbytes.group(1))


def copy_calibration(mib: int, dev) -> None:
    """A plain copy-like kernel of known traffic (reads and writes `mib` MiB once each), run three
    times so that a counter pass over this program can scale FETCH_SIZE / WRITE_SIZE."""
    n = mib * 2**20 // 4
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


# ---------------------------------------------------------------------------------------------

def to_dev(x, dev):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def device_args(inp, dev):
    kw = dict(cu_seqlens_q=to_dev(inp.cu_seqlens_q, dev), cu_seqlens_k=to_dev(inp.cu_seqlens_k, dev),
              seqused_k=to_dev(inp.seqused_k, dev), block_table=to_dev(inp.block_table, dev),
              max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k,
              q_descale=to_dev(inp.q_descale, dev), k_descale=to_dev(inp.k_descale, dev),
              v_descale=to_dev(inp.v_descale, dev), softmax_scale=inp.softmax_scale, causal=inp.causal,
              window_left=inp.window_left, window_right=inp.window_right)
    return to_dev(inp.q, dev), to_dev(inp.k, dev), to_dev(inp.v, dev), kw


# Runs of back-to-back launches timed for each kernel figure; the median run is reported.
TIMING_WINDOWS = 3

# Decode steps captured in one HIP graph: a model's forward replays its attention layers inside one
# graph, back to back; the launch gap of a graph replay comes once per forward, not per layer.
STEPS_PER_GRAPH = 8


def bench_decode_step(inp, steps: int, warmup: int, dev, path: str = "balanced", num_splits=None):
    """One decode step of `path`:
      "balanced": fa8_fwd_decode_scheduled (which derives the per-request split schedule on the
                  device) + fa8_combine_scheduled;
      "static":   fa8_fwd_decode_splitkv with the library's split count + fa8_combine.
    Three timings, with the inputs resident in HBM:
      graph_ms: STEPS_PER_GRAPH steps captured once in a HIP graph and replayed until `steps`
                steps have run, wall time / steps, the median of TIMING_WINDOWS such runs (the
                pages time decode as the per-layer attention span of replayed CUDA graphs); the
                replays' output must equal the eager step's bit for bit;
      eager_ms: the same calls issued eagerly, wall time / steps;
      kernel_ms: HIP events on the launch stream around `steps` decode launches issued back to
                back, elapsed time / steps (the median of TIMING_WINDOWS such runs);
      kernel_ms_events (median, quartiles): HIP events around the decode kernel of every step of the
                eager loop (mean; median and quartiles beside it).
    Returns a dict."""
    q, k, v, kw = device_args(inp, dev)
    B, HQ, SQ, DV = inp.batch, inp.heads_q, inp.max_seqlen_q, inp.dv
    out = torch.empty((q.shape[0], HQ, DV), dtype=torch.bfloat16, device=dev)
    cu = kw["cu_seqlens_q"]
    if path == "balanced":
        W = binding.decode_num_workers(q, k, v, **kw)
        sched = torch.empty(int(binding.load().fa8_decode_schedule_bytes(B)) // 4, dtype=torch.int32, device=dev)
        op = torch.empty((W + B, SQ, HQ, DV), dtype=torch.float32, device=dev)
        lp = torch.empty((W + B, SQ, HQ), dtype=torch.float32, device=dev)

        def pre():
            pass

        def decode():
            binding.decode_scheduled(q, k, v, num_workers=W, schedule=sched, o_partial=op, lse_partial=lp, **kw)

        def post():
            binding.combine_scheduled(op, lp, sched, num_workers=W, batch=B, max_seqlen_q=SQ, heads_q=HQ, dv=DV,
                                      out=out, cu_seqlens_q=cu)
        count = {"num_workers": W}
    else:
        S = num_splits or binding.decode_num_splits_for(q, k, v, **kw)
        op = torch.empty((S, B, SQ, HQ, DV), dtype=torch.float32, device=dev)
        lp = torch.empty((S, B, SQ, HQ), dtype=torch.float32, device=dev)

        def pre():
            pass

        def decode():
            binding.decode_splitkv(q, k, v, num_splits=S, o_partial=op, lse_partial=lp, **kw)

        def post():
            binding.combine(op, lp, batch=B, max_seqlen_q=SQ, heads_q=HQ, dv=DV, out=out, cu_seqlens_q=cu)
        count = {"num_splits": S}

    def step():
        pre()
        decode()
        post()

    for _ in range(warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        pre()
        a.record()
        decode()
        b.record()
        post()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    kt = np.array([a.elapsed_time(b) for a, b in evs])
    # the decode kernel's average launch duration: `steps` launches issued back to back between
    # one pair of events on the launch stream (an event pair around each launch also holds that
    # launch's dispatch latency, a few microseconds)
    # (TIMING_WINDOWS such runs, the median one reported)
    runs = []
    for _ in range(TIMING_WINDOWS):
        ba, bb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ba.record()
        for _ in range(steps):
            decode()
        bb.record()
        torch.cuda.synchronize()
        runs.append(ba.elapsed_time(bb) / steps)
    batched_ms = float(np.median(runs))
    ref = out.clone()
    assert torch.isfinite(ref.float()).all(), "non-finite decode output"
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        for _ in range(STEPS_PER_GRAPH):
            step()
    replays = max(1, -(-steps // STEPS_PER_GRAPH))
    for _ in range(max(1, warmup // STEPS_PER_GRAPH)):
        graph.replay()
    gruns = []
    for _ in range(TIMING_WINDOWS):      # the median of TIMING_WINDOWS runs of `replays` replays
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(replays):
            graph.replay()
        torch.cuda.synchronize()
        gruns.append((time.perf_counter() - t0) * 1e3 / (replays * STEPS_PER_GRAPH))
    graph_ms = float(np.median(gruns))
    assert torch.equal(out, ref), "graph replay differs from the eager decode step"
    res = dict(count, graph_ms=graph_ms, eager_ms=eager_ms, kernel_ms=batched_ms, kernel_ms_events=float(kt.mean()),
               kernel_ms_median=float(np.median(kt)), kernel_ms_q1=float(np.percentile(kt, 25)),
               kernel_ms_q3=float(np.percentile(kt, 75)))
    del graph
    return res


def decode_kernel_name(inp, dev, balanced: bool) -> str:
    """Name of the decode kernel the library's plan picks for this workload."""
    q, k, v, kw = device_args(inp, dev)
    plan = binding.decode_plan(q, k, v, num_splits=1, **kw)
    paged = inp.block_table is not None
    how = "balanced schedule" if balanced else "static splits"
    if plan["kernel"] == 1:
        step_page = (not paged) or inp.page_size >= plan["block_keys"]
        return (f"fa8_decode_heads_kernel<{inp.d},{inp.dv},{plan['heads_per_workgroup']},{int(paged)},{int(step_page)},"
                f"{int(balanced)}> (split-KV decode, {plan['heads_per_workgroup']} kv heads per wave, {how})")
    return f"fa8_decode_kernel<{inp.d},{inp.dv},...,{int(balanced)}> (split-KV decode, one kv head per wave, {how})"


def decode_figures(inp, r: dict) -> dict:
    """GB/s of a bench_decode_step result: the step (graph-replayed and eager) on the step's
    algorithmic bytes, the kernel on the kernel's."""
    sb, kb = decode_step_bytes(inp), decode_kernel_bytes(inp)
    gbs = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9, 2)
    d = {k: v for k, v in r.items() if k in ("num_workers", "num_splits")}
    d.update(step_value=gbs(sb, r["graph_ms"]), step_ms=round(r["graph_ms"], 5),
             step_timing=f"decode (with its split schedule) and combine, {STEPS_PER_GRAPH} steps per HIP graph, "
                         f"replayed back to back",
             eager_step_value=gbs(sb, r["eager_ms"]), eager_step_ms=round(r["eager_ms"], 5),
             kernel_value=gbs(kb, r["kernel_ms"]), kernel_ms=round(r["kernel_ms"], 5),
             kernel_timing=KERNEL_TIMING,
             kernel_ms_per_launch_events={"mean": round(r["kernel_ms_events"], 5),
                                          "median": round(r["kernel_ms_median"], 5),
                                          "quartiles": [round(r["kernel_ms_q1"], 5), round(r["kernel_ms_q3"], 5)]},
             kernel_pct_of_hbm_peak=round(100 * kb / (r["kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2))
    return d


FLUSH_MIB = 512   # more than the L2s and the 256 MB MALL together
KERNEL_TIMING = ("HIP events on the launch stream around the timed launches issued back to back: "
                 "elapsed time / launches, the median of 3 such runs (per-launch event pairs, which "
                 "also hold each launch's dispatch latency, are reported beside it)")


def bench_prefill(inp, steps: int, warmup: int, dev, flushed: bool = False):
    """Prefill launches after `warmup` untimed ones (inputs resident in HBM, caches warm from the
    previous launches). Returns (wall_ms, kernel_ms, event_ms, flushed_ms):
      wall_ms, kernel_ms: `steps` launches issued back to back; wall time per launch (synchronize
          before and after) and the average launch duration from one pair of HIP events around the
          run on the launch stream, for the run with the median kernel time of TIMING_WINDOWS;
      event_ms: the mean of an event pair around each of `steps` more launches (each also holds
          its launch's dispatch latency);
      flushed_ms (with `flushed`, else None): the same per-launch event mean over `steps` launches
          each preceded by a FLUSH_MIB write that evicts the caches (the write is outside the
          events), to compare with event_ms."""
    q, k, v, kw = device_args(inp, dev)
    if getattr(inp, "sink", None) is not None:
        kw["sink"] = to_dev(np.asarray(inp.sink, np.float32), dev)
    odt = torch.float16 if inp.out_dtype == "fp16" else torch.bfloat16
    out = torch.empty(tuple(q.shape[:-1]) + (inp.dv,), dtype=odt, device=dev)
    for _ in range(warmup):
        binding.prefill(q, k, v, out=out, **kw)
    # TIMING_WINDOWS runs of `steps` back-to-back launches; the run with the median kernel time
    # is reported (one run alone can catch a transient slowdown of the whole GPU)
    wins = []
    for _ in range(TIMING_WINDOWS):
        ra, rb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ra.record()
        for _ in range(steps):
            binding.prefill(q, k, v, out=out, **kw)
        rb.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        wins.append((ra.elapsed_time(rb) / steps, (t1 - t0) * 1e3 / steps))
    kernel_ms, wall_ms = sorted(wins)[len(wins) // 2]
    assert torch.isfinite(out.float()).all(), "non-finite prefill output"
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        binding.prefill(q, k, v, out=out, **kw)
        b.record()
    torch.cuda.synchronize()
    event_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    flushed_ms = None
    if flushed:
        buf = torch.empty(FLUSH_MIB << 20, dtype=torch.uint8, device=dev)
        fevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in fevs:
            buf.zero_()
            a.record()
            binding.prefill(q, k, v, out=out, **kw)
            b.record()
        torch.cuda.synchronize()
        flushed_ms = float(np.mean([a.elapsed_time(b) for a, b in fevs]))
        del buf
    return wall_ms, kernel_ms, event_ms, flushed_ms


def bench_prefill_mx(inp, steps: int, warmup: int, dev):
    """Average launch duration of the MXFP8 prefill on an MX-encoded input: one pair of HIP events
    around `steps` back-to-back launches."""
    q, k, v = (to_dev(x, dev) for x in (inp.q, inp.k, inp.v))
    qs, ks, vs = (to_dev(x, dev) for x in (inp.q_mx, inp.k_mx, inp.v_mx))
    out = torch.empty(tuple(q.shape[:-1]) + (inp.dv,), dtype=torch.bfloat16, device=dev)
    kw = dict(causal=inp.causal, window_left=inp.window_left, window_right=inp.window_right, out=out)
    for _ in range(warmup):
        binding.prefill_mx(q, k, v, qs, ks, vs, **kw)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        binding.prefill_mx(q, k, v, qs, ks, vs, **kw)
    b.record()
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "non-finite MX prefill output"
    return a.elapsed_time(b) / steps


def other_workloads(args, dev) -> dict:
    """Figures of the remaining measured workloads, reported beside the headline (not part of
    `value`): the paged GQA decode with the static splits of fa8_fwd_decode_splitkv; long-KV
    decode (4 sequences of 131072 keys, 8/1 heads, 64-token pages; GB/s of the decode step, as a
    replayed HIP graph and eager, and of its kernel) on both paths; the causal prefill workload
    with a learnable sink, the Q quantizer, the MXFP8 prefill on the causal prefill shape, and the
    mixed-shape varlen prefill (8 sequences, window 1024, fp16 out; TFLOP/s of the visible pairs)
    for (d, dv) = (256, 256) and (192, 128)."""
    out = {}
    dec = gen.paged_gqa_decode(1)
    st = bench_decode_step(dec, args.steps, args.warmup // 2, dev, "static", args.num_splits or None)
    out["paged_gqa_decode_static_splits"] = dict(workload=dec.name, unit="GB/s", **decode_figures(dec, st))
    lk = gen.long_kv_decode(3)
    for path in ("balanced", "static"):
        r = bench_decode_step(lk, max(10, args.steps // 2), max(10, args.warmup // 2), dev, path)
        out[f"long_kv_decode_{path}"] = dict(workload=lk.name, unit="GB/s", **decode_figures(lk, r))
    # the causal prefill workload with a learnable sink logit per query head (N(0, 1))
    cs = gen.with_sink(gen.causal_prefill(2), 12)
    ms, kms, _, _ = bench_prefill(cs, max(5, args.prefill_steps // 2), args.prefill_warmup, dev)
    fl = prefill_flop(cs)
    out["causal_prefill_with_sink"] = {"workload": cs.name, "unit": "TFLOP/s",
                                       "kernel_value": round(fl / (kms * 1e-3) / 1e12, 2), "kernel_ms": round(kms, 5),
                                       "kernel_pct_of_fp8_peak": round(100 * fl / (kms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 2)}
    # the Q quantizer (the step before the path) on the causal prefill workload's Q, from bf16
    gq = torch.Generator().manual_seed(13)
    qb = torch.randn((2, 8192, 32, 128), generator=gq).to(torch.bfloat16).to(dev)
    q8 = torch.empty(qb.shape, dtype=torch.uint8, device=dev)
    qs = torch.empty((2, 8), dtype=torch.float32, device=dev)
    for _ in range(10):
        binding.quantize_q(qb, 8, out=q8, descale=qs)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        binding.quantize_q(qb, 8, out=q8, descale=qs)
        b.record()
    torch.cuda.synchronize()
    qms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    qbytes = qb.numel() * 3 + qs.numel() * 4          # bf16 read once, E4M3 written once, descales
    out["q_quantize_causal_prefill"] = {"workload": "q bf16 [2, 8192, 32, 128], 8 kv heads", "unit": "GB/s",
                                        "kernel_value": round(qbytes / (qms * 1e-3) / 1e9, 2), "kernel_ms": round(qms, 5),
                                        "kernel_pct_of_hbm_peak": round(100 * qbytes / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                                        "note": "two launches (block maxima, then codes): Q is read twice"}
    del qb, q8
    # the MXFP8 variant on the causal prefill shape: N(0,1) data encoded as MXFP8 (E4M3 elements,
    # E8M0 scales per 32 elements of d for Q/K and per 32 keys for V)
    mx = gen.make_mx(2, 2, 8192, 8192, 32, 8, 128, 128, causal=True, name="mxfp8_causal_prefill_b2_s8192_h32x8_d128")
    kms = bench_prefill_mx(mx, max(5, args.prefill_steps // 2), args.prefill_warmup, dev)
    fl = prefill_flop(mx)
    out["mxfp8_causal_prefill"] = {"workload": mx.name, "unit": "TFLOP/s",
                                   "kernel_value": round(fl / (kms * 1e-3) / 1e12, 2), "kernel_ms": round(kms, 5),
                                   "kernel_pct_of_fp8_peak": round(100 * fl / (kms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 2)}
    del mx
    for d, dv in ((256, 256), (192, 128)):
        mv = gen.mixed_varlen(4, d=d, dv=dv)
        # twice the causal prefill's warm-up: on a new set of buffers these short launches keep
        # getting faster for the first 100-200 launches (measured in blocks of 20: d = 256 264,
        # 247, 240, 233, 229 us, then about 228; (192, 128) 174 ... 139 us after 200; the causal
        # prefill settles after about 60). A cache-evicting write before each launch does not
        # bring that back, so it is not the caches' contents
        ms, kms, ems, fms = bench_prefill(mv, args.prefill_steps, 2 * args.prefill_warmup, dev, flushed=True)
        fl = prefill_flop(mv)
        out[f"mixed_varlen_d{d}x{dv}"] = {"workload": mv.name, "unit": "TFLOP/s",
                                          "kernel_value": round(fl / (kms * 1e-3) / 1e12, 2), "kernel_ms": round(kms, 5),
                                          "kernel_pct_of_fp8_peak": round(100 * fl / (kms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 2),
                                          "kernel_timing": KERNEL_TIMING,
                                          "per_launch_event_ms": round(ems, 5),
                                          "flushed_kernel_value": round(fl / (fms * 1e-3) / 1e12, 2),
                                          "flushed_kernel_ms": round(fms, 5),
                                          "flushed_note": f"each launch after a {FLUSH_MIB} MiB write (caches cold), an event "
                                                          f"pair around each launch: compare with per_launch_event_ms",
                                          "flop": fl}
    return out


# The decode steps timed on the Hopper FP8 page ("Native FP8 (E4M3 Q/K/V) forward for Hopper",
# Performance, decode table: H200 with locked clocks, vLLM's decode launches replayed as CUDA
# graphs, paged K/V, max_seqlen_k = 32768, the per-layer attention span including the split-KV
# combine, in microseconds). One rank's heads at the stated tensor parallelism, d = 128, every
# request "N k" = N * 1024 keys long. Another machine's figures: context, not a target.
PAGES_DECODE = [
    # (shape, requests, query tokens per request, keys per request, q heads, kv heads,
    #  FA3 FP8 us, FA4 native FP8 us on H200)
    ("Llama-3.1-8B TP1, 1 x 1, 4k", 1, 1, 4096, 32, 8, 17.0, 11.4),
    ("Llama-3.1-8B TP1, 32 x 1, 2k", 32, 1, 2048, 32, 8, 62.6, 36.2),
    ("Llama-3.1-8B TP1, 128 x 1, 1k", 128, 1, 1024, 32, 8, 123.1, 74.8),
    ("Llama-3.1-8B TP1, 16 x 1, 16k", 16, 1, 16384, 32, 8, 189.4, 143.4),
    ("Llama-3.1-8B TP1, 32 x 4, 4k", 32, 4, 4096, 32, 8, 106.1, 66.1),
    ("Llama-3.1-70B TP4, 64 x 1, 4k", 64, 1, 4096, 16, 2, 58.5, 40.4),
    ("Llama-3.1-70B TP4, 8 x 1, 32k", 8, 1, 32768, 16, 2, 57.9, 39.4),
    ("Qwen3-32B TP2, 32 x 1, 8k", 32, 1, 8192, 32, 4, 102.8, 70.6),
]
# The table's two Gemma-4-31B rows (TP4, d = 256, 1024-key window; the page gives no head counts,
# so they are not run): (shape, FA3 FP8 us, FA4 native FP8 us on H200)
PAGES_DECODE_NOT_RUN = [
    ("Gemma-4-31B TP4, 4 x 4, 28k", 23.6, 11.4),
    ("Gemma-4-31B TP4, 16 x 4, 28k", 44.1, 17.0),
]
# K/V pools cycled through by consecutive steps, at least this many MiB in all, so that every
# step reads its K and V from HBM (the page flushes the L2 between layers; here the L2s and the
# 256 MB memory-side cache would otherwise hold the smaller shapes' K/V from one step to the next)
PAGES_ROTATE_MIB = 1024


def pages_decode_shapes(dev, replays: int = 8) -> list:
    """The decode shapes of PAGES_DECODE on this GPU: one decode step = the balanced decode and
    its combine (16-token pages, a random page permutation, descales in [0.5, 2], causal among a
    request's query tokens), captured in a HIP graph of at least 16 steps whose consecutive steps
    read distinct copies of the K/V pools, replayed back to back; wall time per step."""
    rows = []
    for idx, (shape, nreq, nq, keys, hq, hkv, fa3_us, fa4_us) in enumerate(PAGES_DECODE):
        inp = gen.make_paged(40 + idx, [keys] * nreq, hq, hkv, 128, 128, 16, sq=nq, varlen_q=True, causal=nq > 1,
                             descales=(("uniform", 0.5, 2.0),) * 3, max_seqlen_k=32768, name=shape)
        q, k, v, kw = device_args(inp, dev)
        pool = k.numel() + v.numel()
        copies = int(min(64, max(2, -(-PAGES_ROTATE_MIB * 2 ** 20 // pool))))
        ks = [k] + [k.clone() for _ in range(copies - 1)]
        vs = [v] + [v.clone() for _ in range(copies - 1)]
        B, HQ, SQ, DV = inp.batch, inp.heads_q, inp.max_seqlen_q, inp.dv
        W = binding.decode_num_workers(q, k, v, **kw)
        sched = torch.empty(int(binding.load().fa8_decode_schedule_bytes(B)) // 4, dtype=torch.int32, device=dev)
        op = torch.empty((W + B, SQ, HQ, DV), dtype=torch.float32, device=dev)
        lp = torch.empty((W + B, SQ, HQ), dtype=torch.float32, device=dev)
        out = torch.empty((q.shape[0], HQ, DV), dtype=torch.bfloat16, device=dev)

        def step(i):
            binding.decode_scheduled(q, ks[i], vs[i], num_workers=W, schedule=sched, o_partial=op, lse_partial=lp,
                                     **kw)
            binding.combine_scheduled(op, lp, sched, num_workers=W, batch=B, max_seqlen_q=SQ, heads_q=HQ, dv=DV,
                                      out=out, cu_seqlens_q=kw["cu_seqlens_q"])
        for i in range(copies):
            step(i)
        torch.cuda.synchronize()
        ref = out.clone()
        assert torch.isfinite(ref.float()).all(), f"{shape}: non-finite decode output"
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        nsteps = max(copies, 16)    # at least 16 steps per replay, cycling through the copies
        with torch.cuda.graph(graph):
            for i in range(nsteps):
                step(i % copies)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(replays):
            graph.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / (replays * nsteps)
        # every copy holds the same values, so every step's output is the eager one's
        assert torch.equal(out, ref), f"{shape}: graph replay differs from the eager decode step"
        nbytes = decode_step_bytes(inp)
        rows.append({"shape": shape, "step_us": round(us, 2), "num_workers": W,
                     "step_GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "step_bytes": nbytes, "kv_copies": copies,
                     "page_fa4_native_fp8_h200_us": fa4_us, "page_fa3_fp8_h200_us": fa3_us,
                     "page_fa4_us_over_this_us": round(fa4_us / us, 3)})
        del graph, ks, vs, q, k, v, op, lp, out, sched
        torch.cuda.empty_cache()
    return rows


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline_decode(inp, budget_s: float):
    """The oracle (fp64 C, OpenMP on the host cores) on a bounded sample of the decode workload:
    all query heads of the first few sequences, grown until about budget_s of CPU time."""
    import oracle
    cores = host_cores()
    oracle.attention(inp, rows=(np.zeros(1, np.int32), np.zeros(1, np.int32), np.zeros(1, np.int32)), threads=cores)
    rb_all, rh_all, ri_all = oracle.all_rows(inp)
    sk = inp.seqlens_k()
    nb, elapsed, reps = 1, 0.0, 1
    while True:
        sel = rb_all < nb
        t0 = time.perf_counter()
        oracle.attention(inp, rows=(rb_all[sel], rh_all[sel], ri_all[sel]), threads=cores)
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s / 3 or nb >= inp.batch:
            break
        nb = min(inp.batch, max(nb + 1, int(nb * min(8.0, budget_s / 3 / max(elapsed, 1e-3)))))
    if nb >= inp.batch and elapsed < budget_s / 2:
        # the whole workload is quicker than the budget: repeat it for a steadier rate
        reps = max(1, int(budget_s / 2 / max(elapsed, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.attention(inp, rows=(rb_all, rh_all, ri_all), threads=cores)
        elapsed = (time.perf_counter() - t0) / reps
    # bytes of the sampled sequences, as counted for the GPU step
    kv = int(sk[:nb].sum()) * inp.heads_kv * (inp.d + inp.dv)
    frac = nb / inp.batch
    nbytes = kv + frac * (decode_step_bytes(inp) - int(sk.sum()) * inp.heads_kv * (inp.d + inp.dv))
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{nb} of {inp.batch} sequences (all {inp.heads_q} query heads), {elapsed:.2f} s per pass "
                      f"(mean of {reps}) on {cores} threads of {cpu_model()}"}


def cpu_baseline_prefill(inp, budget_s: float):
    """The oracle on every `stride`-th query row of every (batch, head) of the causal prefill
    workload, scaled by the visible pairs it covered."""
    import oracle
    cores = host_cores()
    rb_all, rh_all, ri_all = oracle.all_rows(inp)
    stride = 4096
    while True:
        sel = (ri_all % stride) == (stride - 1)
        rows = (rb_all[sel], rh_all[sel], ri_all[sel])
        t0 = time.perf_counter()
        oracle.attention(inp, rows=rows, threads=cores)
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s / 3 or stride <= 8:
            break
        stride = max(8, int(stride / min(8.0, budget_s / 3 / max(elapsed, 1e-3))))
    # visible keys of the sampled rows (causal, Sq == Sk): i + 1
    pairs = int((rows[2].astype(np.int64) + 1).sum())
    flop = pairs * 2 * (inp.d + inp.dv)
    return {"value": round(flop / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"every {stride}th query row of all heads ({len(rows[0])} rows), {elapsed:.1f} s on {cores} "
                      f"threads of {cpu_model()}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=100,
                    help="untimed launches before each prefill leg (the mixed varlen legs take twice as many)")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="static splits of the paged GQA decode figure beside the headline (0 = the library's heuristic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the long-KV decode and mixed varlen figures")
    ap.add_argument("--no-pages", action="store_true",
                    help="skip the decode shapes of the Hopper FP8 page's table (context figures)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time per workload")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a copy kernel of MIB MiB (for scaling counter passes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this FP8 attention forward has no multi-GPU path "
              "(each GPU would run the same kernels on its own share of heads or pages)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    binding.load()
    if args.calibrate_copy > 0:
        copy_calibration(args.calibrate_copy, dev)

    dec = gen.paged_gqa_decode(1)
    r = bench_decode_step(dec, args.steps, args.warmup, dev, "balanced")
    fig = decode_figures(dec, r)
    step_bytes = decode_step_bytes(dec)
    kbytes = decode_kernel_bytes(dec)
    value = fig["step_value"]
    achieved = fig["kernel_value"]
    line = {
        "metric": "FP8 attn fwd TFLOP/s (prefill) & decode HBM GB/s, % of MI355X peak",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fig["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": dec.name, "batch": dec.batch, "heads_q": dec.heads_q, "heads_kv": dec.heads_kv,
                   "d": dec.d, "page_size": dec.page_size, "seqlens_k": "uniform [1024, 8192], seed 1",
                   "sum_seqlen_k": int(dec.seqlens_k().sum()), "num_workers": r["num_workers"],
                   "split_schedule": "balanced (device-computed per-request splits)", "out": "bf16",
                   "step_bytes": step_bytes, "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "step_timing": fig["step_timing"], "eager_step_value": fig["eager_step_value"],
                   "eager_step_ms": fig["eager_step_ms"]},
        "roofline": {"bound": "hbm", "kernel": decode_kernel_name(dec, dev, True),
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(f"fa8_decode_heads_kernel_balanced_{dec.name}_traffic.md"),
                     "kernel_ms": fig["kernel_ms"], "kernel_timing": KERNEL_TIMING,
                     "kernel_ms_per_launch_events": fig["kernel_ms_per_launch_events"], "bytes_per_launch": kbytes},
    }
    if not args.no_prefill:
        pre = gen.causal_prefill(2)
        p_ms, p_kern, p_events, p_flushed = bench_prefill(pre, args.prefill_steps, args.prefill_warmup, dev, flushed=True)
        flop = prefill_flop(pre)
        tfl = flop / (p_ms * 1e-3) / 1e12
        ktfl = flop / (p_kern * 1e-3) / 1e12
        line["prefill"] = {
            "workload": pre.name, "value": round(tfl, 2), "unit": "TFLOP/s", "ms_per_step": round(p_ms, 4),
            "steps": args.prefill_steps, "flop_per_step": flop, "pct_of_fp8_peak": round(100 * tfl / FP8_PEAK_TFLOPS, 2),
            "roofline": {"bound": "mfma", "kernel": "fa8_prefill_kernel<128,128,64,false> (prefill, contiguous K/V, 64-key tiles)",
                         "achieved": round(ktfl, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ktfl / FP8_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic(f"fa8_prefill_kernel_{pre.name}_traffic.md"),
                         "kernel_ms": round(p_kern, 4), "kernel_timing": KERNEL_TIMING,
                         "kernel_ms_per_launch_events": round(p_events, 4)},
            "flushed_kernel_ms": round(p_flushed, 4),
            "flushed_kernel_value": round(flop / (p_flushed * 1e-3) / 1e12, 2),
            "flushed_note": f"each launch after a {FLUSH_MIB} MiB write (caches cold), an event pair around each "
                            f"launch: compare with kernel_ms_per_launch_events",
        }
    if not args.no_extra:
        line["other_workloads"] = other_workloads(args, dev)
    if not args.no_pages:
        line["pages_decode_shapes"] = {
            "note": "the decode steps of the Hopper FP8 page's decode table on this GPU (balanced decode + combine, "
                    "graph-replayed, K/V read from HBM every step), the page's H200 times beside them as context "
                    "from another machine",
            "shapes": pages_decode_shapes(dev)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(dec, args.cpu_budget)
        if "prefill" in line:
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(gen.causal_prefill(2), args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
