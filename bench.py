#!/usr/bin/env python3
"""Throughput of the quantized-attention path on one MI355X.

Headline (``value``): the SageAttention-style varlen prefill workload --
B=8, lengths U{512..4096} (seeded), causal, 32 q / 8 kv heads, D=128, fp16
Q/K/V with 1% offset channels -- one step = per-block int8 quant of Q and K
+ transposed/permuted fp16 V + int8-QK / fp16-PV prefill, all inputs already
in HBM.  value = algorithmic attention FLOP of the step / step time, in
TFLOP/s (4 * D * H_q * sum over sequences of L(L+1)/2).

Also reported (``extra``): the paged fp8 decode (GB/s of K/V bytes), the
long fp8 prefill with RoPE + paged append (TFLOP/s), the sparse MLA decode
(GB/s) and a chunked prefill against a paged bf16 cache (TFLOP/s of the
prefill alone and of page gather + quantization + prefill), each timed on
its own, each with the oracle timed beside it on a bounded sample.

``roofline``: the prefill kernel alone, timed with HIP events on the stream
it is launched on, against the MFMA peak of its two contractions (int8 QK at
5.0 POP/s, fp16 PV at 2.5 PFLOP/s: 2 / (1/5000 + 1/2500) = 3333 TFLOP/s for
equal flop counts).  ``traffic``: HBM-side bytes of one launch from two
rocprofv3 counter runs of ``bench.py --traffic-probe`` (FETCH_SIZE, then
WRITE_SIZE), each scaled by what the same counter reads for a device copy of
known size; ``bench.py --summarize-traffic`` stores them under profiles/
with a hash of the kernel sources, and the figure is reported only while
that hash matches.  ``cpu_baseline``: the fp64 oracle on a bounded sample
of the same workload, on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill TFLOPS (% FP8 MFMA peak); decode HBM GB/s (% of peak)"
PEAK_FP8 = 5000.0        # TFLOP/s dense
PEAK_I8 = 5000.0         # TOP/s dense
PEAK_F16 = 2500.0        # TFLOP/s dense
PEAK_HBM = 8000.0        # GB/s


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_prefill_sage_varlen.md")
TRAFFIC_SOURCES = ("paged_kv_amd/csrc/prefill.hip", "paged_kv_amd/csrc/kcommon.h", "paged_kv_amd/csrc/launch.h")
CALIB_BYTES = 256 << 20  # device-to-device copy used to scale the counters


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(lens) -> int:
    return int(sum(int(L) * (int(L) + 1) // 2 for L in lens))


def time_events(fn, iters, flush=None):
    """Per-call durations (ms) of fn() with events on the current stream.  The
    calls (and the untimed flush before each) are queued back to back and
    synchronized once, so the GPU never idles between them."""
    import torch
    ev = []
    for _ in range(iters):
        if flush is not None:
            flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        ev.append((s, e))
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def settle(fn, min_ms=250.0):
    """Runs fn back to back (untimed) until min_ms of GPU time has passed.  An
    idle GPU's clocks take some 50 ms of load to reach their sustained level
    (measured: the config-2 step falls from 0.64 to 0.52 ms over the first
    ~50 ms, then stays flat); a measurement taken earlier reports the ramp."""
    import torch
    total = 0.0
    while total < min_ms:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(4):
            fn()
        e.record()
        e.synchronize()
        total += s.elapsed_time(e)
    return total


def make_flush():
    """Reads a 1 GiB buffer: evicts L2 and the 256 MB Infinity Cache with
    clean lines.  (Writing it instead left dirty lines whose write-back then
    competed with the timed call: ~60 us on the config-3 decode.)"""
    import torch
    buf = torch.ones(1 << 29, dtype=torch.float16, device="cuda")
    return lambda: buf.sum(dtype=torch.float32)


def bench_config2(steps, warmup):
    import torch
    import gen
    from paged_kv_amd.pipeline import SagePrefill
    from tests.parity import to_dev
    x = gen.config2()
    lens = x["seqlens"]
    p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["cu_seqlens"]),
                    int(lens.max()), x["sm_scale"], causal=True)
    flops = 4.0 * 128 * 32 * causal_pairs(lens)
    settle_ms = settle(p.run)
    for _ in range(warmup):
        p.run()
    torch.cuda.synchronize()
    # timed region: every step is quantize + prefill.  Events on the launch
    # stream bracket the prefill launch of every SAMPLE-th step, so its
    # duration is taken in the same back-to-back run that gives the step time
    # (an event pair leaves a gap of ~6 us between kernels: sampled, not on
    # every step)
    SAMPLE = 4
    picked = list(range(0, steps, SAMPLE))
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in picked}
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s.record()
    for i in range(steps):
        p.quantize()
        if i in ev:
            ev[i][0].record()
        p.attend()
        if i in ev:
            ev[i][1].record()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = s.elapsed_time(e) / steps
    kms = [ev[i][0].elapsed_time(ev[i][1]) for i in picked]
    kavg = float(np.mean(kms))
    qms = time_events(p.quantize, 10)  # the quantization alone (after the timed region)
    # the same flow with SageAttention's K smoothing (per-sequence channel
    # means subtracted before the int8 blocks): not the headline step, which
    # is plain amax/127 quantization
    ps = SagePrefill(p.q, p.k, p.v, p.cu, p.max_seqlen, x["sm_scale"], causal=True, smooth_k=True)
    sq = time_events(ps.quantize, 10)
    sr = time_events(ps.run, 10)
    del ps
    # and with fp8 V under per-channel descales as well
    pr = SagePrefill(p.q, p.k, p.v, p.cu, p.max_seqlen, x["sm_scale"], causal=True, smooth_k=True,
                     v_fp8_per_channel=True)
    rq = time_events(pr.quantize, 10)
    rr = time_events(pr.run, 10)
    ra = time_events(pr.attend, 10)
    del pr
    return {
        "x": x, "lens": lens, "flops": flops, "ms_per_step": ms, "wall_s": wall,
        "kernel_ms": kavg, "kernel_ms_min": float(np.min(kms)), "quant_ms": float(np.mean(qms)),
        "settle_ms": settle_ms, "smooth_k_quant_ms": float(np.mean(sq)), "smooth_k_step_ms": float(np.mean(sr)),
        "refined_quant_ms": float(np.mean(rq)), "refined_step_ms": float(np.mean(rr)),
        "refined_prefill_ms": float(np.mean(ra)),
    }


def bench_config3(iters, cpu=False):
    import torch
    import gen
    from paged_kv_amd.pipeline import PagedDecode
    from tests.parity import to_dev
    x = gen.config3()
    p = PagedDecode(to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(x["k_scale"]),
                    to_dev(x["v_scale"]), to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]),
                    to_dev(x["kv_last_page_len"]), x["max_kv_len"], x["sm_scale"])
    kv_bytes = float(np.sum(x["kv_lens"].astype(np.int64)) * 8 * 128 * 2)
    other = 64 * 32 * 128 * 2 * 2 + x["kv_indices"].size * 4 + 65 * 4 * 2
    settle(p.run)
    ms = time_events(p.run, iters, make_flush())
    med = float(np.median(ms))
    gbs = (kv_bytes + other) / (med * 1e-3) / 1e9
    r = {"ms": med, "ms_min": float(np.min(ms)), "bytes": kv_bytes + other, "GB/s": gbs,
         "pct_hbm": 100 * gbs / PEAK_HBM}
    if cpu:
        r["cpu_oracle"] = oracle_config3(x)
    return r


def bench_config5(iters, cpu=False):
    import torch
    import gen
    from paged_kv_amd.pipeline import AppendRopeFp8Prefill
    from tests.parity import to_dev
    x = gen.config5()
    ps = x["page_size"]
    kc = torch.zeros((x["num_pages"], ps, 64, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q0, k0 = to_dev(x["q"]), to_dev(x["k"])
    p = AppendRopeFp8Prefill(q0.clone(), k0.clone(), to_dev(x["v"]), to_dev(x["cu_seqlens"]),
                             to_dev(x["kv_len_before"]), 32768, to_dev(x["rope_cos_sin"]), kc, vc,
                             to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]), ps, x["sm_scale"])
    p.run()
    torch.cuda.synchronize()
    flops = 4.0 * 128 * 64 * causal_pairs([32768])
    settle(p.prefill.attend)
    kms = time_events(p.prefill.attend, iters)
    # whole pipeline: the append rotates q/k in place, so restore them first (untimed)

    def restore():
        p.q.copy_(q0)
        p.k.copy_(k0)
    pipe = time_events(p.run, max(2, iters // 2), restore)
    med = float(np.median(kms))
    r = {"prefill_ms": med, "prefill_TFLOPS": flops / (med * 1e-3) / 1e12,
         "pct_fp8_peak": 100 * flops / (med * 1e-3) / 1e12 / PEAK_FP8,
         "pipeline_ms": float(np.median(pipe)),
         "pipeline_TFLOPS": flops / (np.median(pipe) * 1e-3) / 1e12}
    if cpu:
        r["cpu_oracle"] = oracle_config5(x)
    return r


def bench_config4(iters, cpu=False):
    import torch
    import gen
    from paged_kv_amd.pipeline import SparseMlaDecode
    from tests.parity import to_dev
    x = gen.config4()
    p = SparseMlaDecode(to_dev(x["q"]), to_dev(x["kv_cache"]), to_dev(x["block_table"]),
                        to_dev(x["kv_lens"]), to_dev(x["sparse_indices"]), x["sm_scale"])
    nbytes = 32 * 2048 * 656 + 32 * 128 * 576 * 2 + 32 * 128 * 512 * 2 + 32 * 2048 * 4 + 32 * 1024 * 4
    flops = 32 * 128 * 2048 * 2.0 * (576 + 512)
    p.run()
    torch.cuda.synchronize()
    settle(p.run)
    ms = time_events(p.run, iters, make_flush())
    med = float(np.median(ms))
    gbs = nbytes / (med * 1e-3) / 1e9
    r = {"ms": med, "ms_min": float(np.min(ms)), "bytes": nbytes, "GB/s": gbs,
         "pct_hbm": 100 * gbs / PEAK_HBM, "TFLOPS": flops / (med * 1e-3) / 1e12}
    if cpu:
        r["cpu_oracle"] = oracle_config4(x)
    del p, x
    torch.cuda.empty_cache()
    # the variants at the same size (2048 selected rows of 656 bytes per query row):
    # fp8 e4m3 rows; 128 entries of 16-token blocks
    for name, kw in (("fp8_rows", dict(kv_dtype="fp8")), ("block_sparse_16", dict(sparse_block_size=16))):
        topk = 2048 // kw.get("sparse_block_size", 1)
        y = gen.sparse_mla_inputs(gen.seed_for(4), 32, 1, 128, 65536, 64, topk, **kw)
        pv = SparseMlaDecode(to_dev(y["q"]), to_dev(y["kv_cache"]), to_dev(y["block_table"]),
                             to_dev(y["kv_lens"]), to_dev(y["sparse_indices"]), 1.0 / 24.0,
                             kv_fp8=y["kv_dtype"] == "fp8", sparse_block_size=y["sparse_block_size"])
        pv.run()
        torch.cuda.synchronize()
        settle(pv.run)
        vms = float(np.median(time_events(pv.run, iters, make_flush())))
        vbytes = nbytes - 32 * 2048 * 4 + 32 * topk * 4
        r[name] = {"ms": vms, "GB/s": vbytes / (vms * 1e-3) / 1e9, "pct_hbm": 100 * vbytes / (vms * 1e-3) / 1e9 / PEAK_HBM}
        del pv, y
        torch.cuda.empty_cache()
    return r


def bench_paged_prefill(iters, cpu=False):
    """Chunked prefill against the paged bf16 cache: gather + fp8 quant + prefill."""
    import torch
    import gen
    from paged_kv_amd.pipeline import PagedPrefill
    from tests.parity import to_dev
    x = gen.paged_prefill_workload()
    p = PagedPrefill(to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(x["kv_indptr"]),
                     to_dev(x["kv_indices"]), to_dev(x["kv_last_page_len"]), to_dev(x["cu_q"]),
                     to_dev(x["cu_k"]), x["max_q"], x["max_k"], x["sm_scale"], causal=True)
    p.run()
    torch.cuda.synchronize()
    lq, lk = x["q_lens"].astype(np.int64), x["kv_lens"].astype(np.int64)
    pairs = float(np.sum(lq * (lk - lq) + lq * (lq + 1) // 2))
    flops = 4.0 * 128 * 32 * pairs
    settle(p.attend)
    kms = time_events(p.attend, iters)
    pipe = time_events(p.run, max(2, iters // 2))
    gms = float(np.median(time_events(p.gather, iters)))
    med = float(np.median(kms))
    r = {"prefill_ms": med, "prefill_TFLOPS": flops / (med * 1e-3) / 1e12,
         "pct_fp8_peak": 100 * flops / (med * 1e-3) / 1e12 / PEAK_FP8,
         "pipeline_ms": float(np.median(pipe)),
         "pipeline_TFLOPS": flops / (np.median(pipe) * 1e-3) / 1e12,
         "gathered_bytes": float(2 * np.sum(lk) * 8 * 128 * 2),
         # the page gather alone: every cached K and V row read once and written once
         "gather_ms": gms, "gather_GB/s": 2 * float(2 * np.sum(lk) * 8 * 128 * 2) / (gms * 1e-3) / 1e9}
    if cpu:
        r["cpu_oracle"] = oracle_paged_prefill(x)
    return r


def oracle_paged_prefill(x, budget_s=4.0):
    """The fp64 oracle of the chunked paged prefill: pages read into the
    ragged layout and fp8 quantization first (not timed), then whole
    (sequence, q head) problems in order, in blocks of 256 query rows, until
    the budget is spent; TFLOP/s counts the visible (query, key) pairs done."""
    from oracle.attention import dequant_fp8_per_head, prefill_varlen, ragged_from_pages
    from oracle.quant import quant_fp8_per_head
    tp = time.perf_counter()
    kg = ragged_from_pages(x["k_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], x["cu_k"])
    vg = ragged_from_pages(x["v_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], x["cu_k"])
    qd = dequant_fp8_per_head(*quant_fp8_per_head(x["q"], "bf16"))
    kd = dequant_fp8_per_head(*quant_fp8_per_head(kg, "bf16"))
    vd = dequant_fp8_per_head(*quant_fp8_per_head(vg, "bf16"))
    t_prep = time.perf_counter() - tp
    t, pairs, chunks, done = 0.0, 0, 0, []
    for b in range(len(x["q_lens"])):
        lq, lk = int(x["q_lens"][b]), int(x["kv_lens"][b])
        h = 0
        while h < 32 and t < budget_s:
            for c in range(lq // 256):
                idx = np.arange(c * 256, (c + 1) * 256)
                t0 = time.perf_counter()
                prefill_varlen(qd, kd, vd, x["cu_q"], x["cu_k"], x["sm_scale"], True, "bf16", rows=[(b, h, idx)])
                t += time.perf_counter() - t0
                pairs += int((idx + lk - lq + 1).sum())
                chunks += 1
            h += 1
        done.append(f"{b}:{h}h")
        if t >= budget_s:
            break
    return {"TFLOP/s": 4.0 * 128 * pairs / t / 1e12, "cores": host_cores(), "kind": "oracle",
            "sample": f"whole (sequence, q head) chunks ({' '.join(done)}; {chunks} blocks of 256 query rows, "
                      f"{pairs} causal pairs), fp64 numpy, {t:.1f} s (page reads + quantization "
                      f"{t_prep:.1f} s not counted)"}


def host_cores() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def oracle_config3(x, budget_s=3.0):
    """The fp64 oracle of the paged fp8 decode on whole sequences (all 32 q
    heads), in batch order until the budget is spent; GB/s of fp8 K/V read."""
    from oracle.attention import decode_paged
    lens = x["kv_lens"].astype(np.int64)
    t, nbytes, done = 0.0, 0.0, 0
    while done < len(lens) and t < budget_s:
        t0 = time.perf_counter()
        decode_paged(x["q"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"], x["kv_indptr"],
                     x["kv_indices"], x["kv_last_page_len"], x["sm_scale"], batches=[done])
        t += time.perf_counter() - t0
        nbytes += float(lens[done]) * 8 * 128 * 2
        done += 1
    return {"GB/s": nbytes / t / 1e9, "cores": host_cores(), "kind": "oracle",
            "sample": f"sequences 0..{done - 1} of 64 ({int(lens[:done].sum())} tokens, 32 q heads), "
                      f"fp64 numpy, {t:.1f} s"}


def oracle_config4(x, budget_s=4.0):
    """The fp64 oracle of the sparse MLA decode on whole (sequence, query)
    problems (128 heads, 2048 selected rows), in batch order until the budget
    is spent; GB/s of 656-byte cache rows read."""
    from oracle.attention import sparse_mla_decode, MLA_ROW
    nb = x["q"].shape[0]
    t, rows, done = 0.0, 0, 0
    while done < nb and t < budget_s:
        t0 = time.perf_counter()
        sparse_mla_decode(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"], x["sparse_indices"],
                          x["sm_scale"], batches=[done])
        t += time.perf_counter() - t0
        idx = np.asarray(x["sparse_indices"][done], np.int64)
        rows += int(((idx >= 0) & (idx < int(x["kv_lens"][done]))).sum())
        done += 1
    return {"GB/s": rows * MLA_ROW / t / 1e9, "cores": host_cores(), "kind": "oracle",
            "sample": f"sequences 0..{done - 1} of {nb} ({rows} rows x 128 heads), fp64 numpy, {t:.1f} s"}


def oracle_config5(x, budget_s=4.0):
    """The fp64 oracle of the long causal fp8 prefill for q/kv head 0: RoPE
    and per-head fp8 quantization first (not timed), then chunks of 256 query
    rows drawn at random from the 32768 until the budget is spent; TFLOP/s
    counts the visible (query, key) pairs of the rows done."""
    from oracle.attention import dequant_fp8_per_head, prefill_varlen
    from oracle.quant import quant_fp8_per_head
    from oracle.rope import append_kv_rope
    S, ps = 32768, x["page_size"]
    one = lambda a: np.ascontiguousarray(a[:, :1])
    tp = time.perf_counter()
    zero = np.zeros((x["num_pages"], ps, 1, 128), np.uint16)
    ref = append_kv_rope(one(x["q"]), one(x["k"]), one(x["v"]), "bf16", x["cu_seqlens"], x["kv_len_before"],
                         x["rope_cos_sin"], zero, zero.copy(), x["kv_indptr"], x["kv_indices"], ps)
    qd = dequant_fp8_per_head(*quant_fp8_per_head(ref[0], "bf16"))
    kd = dequant_fp8_per_head(*quant_fp8_per_head(ref[1], "bf16"))
    vd = dequant_fp8_per_head(*quant_fp8_per_head(one(x["v"]), "bf16"))
    t_prep = time.perf_counter() - tp
    cu = np.array([0, S], np.int32)
    rng = np.random.default_rng(55)
    t, pairs, chunks = 0.0, 0, 0
    for c in rng.permutation(S // 256):
        if t >= budget_s:
            break
        idx = np.arange(c * 256, (c + 1) * 256)
        t0 = time.perf_counter()
        prefill_varlen(qd, kd, vd, cu, cu, x["sm_scale"], True, "bf16", rows=[(0, 0, idx)])
        t += time.perf_counter() - t0
        pairs += int((idx + 1).sum())
        chunks += 1
    return {"TFLOP/s": 4.0 * 128 * pairs / t / 1e12, "cores": host_cores(), "kind": "oracle",
            "sample": f"head 0, {chunks} random chunks of 256 query rows ({pairs} causal pairs), fp64 numpy, "
                      f"{t:.1f} s (RoPE + quantization {t_prep:.1f} s not counted)"}


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_probe():
    """One calibration copy of CALIB_BYTES and one headline prefill launch
    (run under rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)."""
    import torch
    import gen
    from paged_kv_amd.pipeline import SagePrefill
    from tests.parity import to_dev
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    x = gen.config2()
    p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["cu_seqlens"]),
                    int(x["seqlens"].max()), x["sm_scale"], causal=True)
    p.quantize()
    torch.cuda.synchronize()
    p.attend()
    torch.cuda.synchronize()
    log("[bench] traffic probe done")


def _counter_rows(d):
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return list(csv.DictReader(open(f[0])))


def summarize_traffic(fetch_dir, write_dir, fetch_cmd, write_cmd):
    """Turn the two counter runs into profiles/traffic_k_prefill_sage_varlen.md."""
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == name]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        pf = [float(r["Counter_Value"]) for r in rows if "k_prefill" in r["Kernel_Name"]]
        if not copies or len(pf) != 1:
            raise SystemExit(f"{name}: expected copy dispatches and one k_prefill dispatch, got {len(copies)}, {len(pf)}")
        calib = max(copies)  # KiB for the CALIB_BYTES copy
        factor = (CALIB_BYTES / 1024.0) / calib
        out[name] = {"kernel_kib": pf[0], "copy_kib": calib, "factor": factor, "bytes": pf[0] * factor * 1024.0}
    traffic = out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]
    import gen
    lens = gen.configs.config2_lengths()
    t, spad = int(lens.sum()), (int(lens.max()) + 127) // 128 * 128
    unique = t * 32 * 128 * 2 + t * 8 * 128 + len(lens) * 8 * 128 * spad * 2 + t * 32 * 128 * 2 \
        + len(lens) * 8 * (spad // 128) * 4
    h = kernel_source_hash()
    lines = [
        "# HBM-side traffic of one k_prefill launch (sage varlen workload: fp16 Q quantized to int8 in",
        "# the kernel, int8 K, fp16 V^T, fp16 O)",
        "",
        "Workload: B=8, lengths U{512..4096} (seed 1002), causal, Hq=32, Hkv=8, D=128; one launch of",
        "`attn_prefill_varlen` (INT8_PER_BLOCK_RAW_Q) after `attn_quant_qk` (K) and",
        "`attn_quant_v_permute` (V) (bench.py --traffic-probe).",
        "",
        f"Unique bytes the launch must move: {unique:.4g} (fp16 Q + int8 K + fp16 V^T with its padding",
        "+ fp16 O + scales), against the measured total below.",
        "",
        "Commands (from the repository root on the GPU host, `cd /tmp && export TMPDIR=/tmp` first):",
        "",
        f"    {fetch_cmd}",
        f"    {write_cmd}",
        "",
        "Calibration: a device-to-device copy of 256 MiB (__amd_rocclr_copyBuffer) moves 262144 KiB each way;",
        "each counter is scaled by 262144 / (its reading for that copy).",
        "",
        "| counter | k_prefill (KiB) | 256 MiB copy (KiB) | factor | k_prefill bytes |",
        "|---|---|---|---|---|",
    ]
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        o = out[name]
        lines.append(f"| {name} | {o['kernel_kib']:.0f} | {o['copy_kib']:.0f} | {o['factor']:.4f} | {o['bytes']:.4g} |")
    lines += ["", f"traffic_bytes_per_launch: {traffic:.6g}", f"kernel_source_hash: {h}", ""]
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps({"traffic_bytes": traffic, "hash": h, **out}))


def stored_traffic():
    """Bytes per launch from the committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = dict(l.split(": ", 1) for l in txt.splitlines() if l.startswith(("traffic_bytes_per_launch", "kernel_source_hash")))
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    return float(vals["traffic_bytes_per_launch"])


def cpu_baseline(x, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the config-2 workload: whole
    (sequence, q head) attention problems, sequence by sequence, added until
    the time budget is spent."""
    from oracle.attention import dequant_int8_per_block, prefill_varlen
    from oracle.quant import quant_int8_per_block, as_f32
    cores = host_cores()
    cu = x["cu_seqlens"]
    t_att, t_prep, flops, done = 0.0, 0.0, 0.0, []
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = s1 - s0
        one = np.array([0, L], np.int32)
        tp = time.perf_counter()
        qc, qs = quant_int8_per_block(x["q"][s0:s1], "fp16", one, L)
        kc, ks = quant_int8_per_block(x["k"][s0:s1], "fp16", one, L)
        qd = dequant_int8_per_block(qc, qs, one)
        kd = dequant_int8_per_block(kc, ks, one)
        vd = as_f32(x["v"][s0:s1], "fp16").astype(np.float64)
        t_prep += time.perf_counter() - tp
        heads = 0
        while heads < 32 and t_att < budget_s:
            ta = time.perf_counter()
            prefill_varlen(qd[:, heads:heads + 1], kd[:, heads // 4:heads // 4 + 1],
                           vd[:, heads // 4:heads // 4 + 1], one, one, x["sm_scale"], True, "fp16")
            t_att += time.perf_counter() - ta
            heads += 1
        flops += 4.0 * 128 * heads * L * (L + 1) / 2
        done.append(f"{b}:L={L}x{heads}h")
        if t_att >= budget_s:
            break
    return {"value": flops / t_att / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"config-2 (sequence:length x q heads) {' '.join(done)}, causal, fp64 numpy; "
                      f"{t_att:.1f} s of attention (quantization {t_prep:.1f} s not counted)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--extra", default="c3,c5,c4,paged", help="comma list of extra workloads (c3,c4,c5,paged) or ''")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run the calibration copy and one prefill launch (for rocprofv3 --pmc)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "FETCH_CMD", "WRITE_CMD"),
                    help="write the traffic summary under profiles/ from two counter runs")
    a = ap.parse_args()
    if a.summarize_traffic:
        summarize_traffic(*a.summarize_traffic)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    import paged_kv_amd
    paged_kv_amd.lib()
    if a.traffic_probe:
        traffic_probe()
        return

    log("[bench] config2 (headline)")
    r2 = bench_config2(a.steps, a.warmup)
    value = r2["flops"] / (r2["ms_per_step"] * 1e-3) / 1e12
    k_tflops = r2["flops"] / (r2["kernel_ms"] * 1e-3) / 1e12
    peak_mixed = 2.0 / (1.0 / PEAK_I8 + 1.0 / PEAK_F16)
    extra = {"config2": {"step_ms": r2["ms_per_step"], "prefill_kernel_ms": r2["kernel_ms"],
                         "prefill_kernel_ms_min": r2["kernel_ms_min"], "quant_ms": r2["quant_ms"],
                         "untimed_settle_ms": r2["settle_ms"],
                         "smooth_k_quant_ms": r2["smooth_k_quant_ms"], "smooth_k_step_ms": r2["smooth_k_step_ms"],
                         "smooth_k_fp8_v_per_channel": {"quant_ms": r2["refined_quant_ms"],
                                                        "prefill_ms": r2["refined_prefill_ms"],
                                                        "step_ms": r2["refined_step_ms"]},
                         "prefill_kernel_TFLOPS": k_tflops, "pct_fp8_peak_step": 100 * value / PEAK_FP8,
                         "pct_fp8_peak_kernel": 100 * k_tflops / PEAK_FP8}}
    for name, fn, it in (("c3", bench_config3, 20), ("c5", bench_config5, 5), ("c4", bench_config4, 30),
                         ("paged", bench_paged_prefill, 10)):
        if name not in a.extra.split(","):
            continue
        log(f"[bench] {name}")
        try:
            extra[{"c3": "config3_decode", "c5": "config5_long_prefill", "c4": "config4_sparse_mla",
                   "paged": "chunked_prefill_paged"}[name]] = \
                fn(it, cpu=not a.no_cpu_baseline)
        except Exception as ex:  # report, keep the headline line
            extra[name] = {"error": f"{type(ex).__name__}: {ex}"}
        torch.cuda.empty_cache()
    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(r2["x"])
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": r2["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8 QK / fp16 PV (fp32 accumulate)",
        "data": "synthetic (seeded)",
        "config": {"workload": "sage_int8_varlen_prefill: B=8, lens U{512..4096} seed 1002, causal, "
                               "Hq=32, Hkv=8, D=128, fp16 in/out; step = int8 quant Q,K + V permute + prefill",
                   "tokens": int(np.sum(r2["lens"])), "lens": [int(v) for v in r2["lens"]],
                   "step_flop": r2["flops"]},
        "pct_fp8_peak": 100 * value / PEAK_FP8,
        "roofline": {"bound": "mfma", "achieved": k_tflops, "peak": peak_mixed, "unit": "TFLOP/s",
                     "frac": k_tflops / peak_mixed, "traffic": stored_traffic(),
                     "kernel": "k_prefill<128, int8 QK, fp16 V>",
                     "per_launch_flop": r2["flops"], "avg_launch_ms": r2["kernel_ms"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
