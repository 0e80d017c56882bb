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
(GB/s), a chunked prefill against a paged bf16 cache (TFLOP/s of the
prefill alone and of page gather + quantization + prefill) and the same
chunks against a paged fp8 cache read inside the prefill kernel (Q
quantization + prefill), each timed on its own, the first four with the
oracle timed beside them on a bounded sample.

``roofline``: the prefill kernel alone, timed with HIP events on the stream
it is launched on, against the MFMA peak of its two contractions (int8 QK at
5.0 POP/s, fp16 PV at 2.5 PFLOP/s: 2 / (1/5000 + 1/2500) = 3333 TFLOP/s for
equal flop counts); the extra workloads carry roofline objects of their own
(decode and sparse MLA against 8 TB/s, the long fp8 prefill against the f16
MFMA peak of its exact QK and PV).  ``traffic``: HBM-side bytes of one
launch from rocprofv3 counter runs of ``bench.py --counter-probe WL``
(FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads for
a device copy of known size; ``bench.py --summarize-counters WL DIR`` writes
them, with the MFMA-busy and instruction-mix passes, to profiles/ together
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
         "pct_hbm": 100 * gbs / PEAK_HBM,
         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s", "frac": gbs / PEAK_HBM,
                      "traffic": stored_counters("c3").get("traffic_bytes_per_launch"),
                      "kernel": "k_decode_split<128> + k_decode_merge<128> (caches evicted before each call)",
                      "per_launch_bytes": kv_bytes + other, "avg_launch_ms": float(np.mean(ms))}}
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
    # the same launch with QK^T on the fp8 matrix instruction (opt-in mode,
    # outside the output tolerance on this workload's outlier rows)
    import paged_kv_amd.api as A
    pf = p.prefill

    def attend_mma8():
        A.attn_prefill_varlen(pf.qc, pf.kc, pf.vp, A.FP8E4M3, A.FP16, pf.qs, pf.ks, pf.vs, A.Q_FP8_PER_HEAD,
                              A.Q_FP8_PER_HEAD_MFMA8, pf.cu, pf.cu, pf.b, pf.max_seqlen, pf.max_seqlen, pf.t, pf.t,
                              pf.hq, pf.hkv, pf.d, pf.sm_scale, pf.causal, pf.o, A.BF16, pf.lse)
    fast = float(np.median(time_events(attend_mma8, iters)))
    tf = flops / (med * 1e-3) / 1e12
    r = {"prefill_ms": med, "prefill_TFLOPS": tf,
         "pct_fp8_peak": 100 * tf / PEAK_FP8,
         "pipeline_ms": float(np.median(pipe)),
         "pipeline_TFLOPS": flops / (np.median(pipe) * 1e-3) / 1e12,
         "prefill_fp8_mfma_qk_ms": fast, "prefill_fp8_mfma_qk_TFLOPS": flops / (fast * 1e-3) / 1e12,
         "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_F16, "unit": "TFLOP/s", "frac": tf / PEAK_F16,
                      "traffic": stored_counters("c5").get("traffic_bytes_per_launch"),
                      "mfma_util_pct": stored_counters("c5").get("mfma_util_pct"),
                      "kernel": "k_prefill<128, fp8 codes summed exactly on f16 MFMA, fp16 V, bf16 O>",
                      "per_launch_flop": flops, "avg_launch_ms": float(np.mean(kms))}}
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
    nbytes = C4_BYTES
    flops = 32 * 128 * 2048 * 2.0 * (576 + 512)
    p.run()
    torch.cuda.synchronize()
    settle(p.run)
    ms = time_events(p.run, iters, make_flush())
    med = float(np.median(ms))
    gbs = nbytes / (med * 1e-3) / 1e9
    r = {"ms": med, "ms_min": float(np.min(ms)), "bytes": nbytes, "GB/s": gbs,
         "pct_hbm": 100 * gbs / PEAK_HBM, "TFLOPS": flops / (med * 1e-3) / 1e12,
         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s", "frac": gbs / PEAK_HBM,
                      "traffic": stored_counters("c4").get("traffic_bytes_per_launch"),
                      "mfma_util_pct": stored_counters("c4").get("mfma_util_pct"),
                      "kernel": "sparse MLA split + merge (caches evicted before each call)",
                      "per_launch_bytes": nbytes, "avg_launch_ms": float(np.mean(ms))}}
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


def bench_paged_prefill_fp8(iters):
    """Chunked prefill against a paged fp8 cache, the pages read inside the
    kernel: fp8 per-head Q quantization + the paged prefill.  The same
    lengths, heads and page size as the bf16-cache flow; Q is that flow's
    bf16 chunk."""
    import torch
    import gen
    from paged_kv_amd.pipeline import PagedPrefillFp8
    from tests.parity import to_dev
    x = gen.paged_prefill_fp8_workload()
    qb = gen.paged_prefill_workload()["q"]
    assert qb.shape == x["q"].shape
    p = PagedPrefillFp8(to_dev(qb), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(x["k_scale"]),
                        to_dev(x["v_scale"]), to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]),
                        to_dev(x["kv_last_page_len"]), to_dev(x["cu_q"]), x["max_q"], x["max_kv_len"],
                        x["sm_scale"], causal=True)
    p.run()
    torch.cuda.synchronize()
    lq, lk = x["q_lens"].astype(np.int64), x["kv_lens"].astype(np.int64)
    pairs = float(np.sum(lq * (lk - lq) + lq * (lq + 1) // 2))
    flops = 4.0 * 128 * 32 * pairs
    settle(p.attend)
    kms = time_events(p.attend, iters)
    pipe = time_events(p.run, max(2, iters // 2))
    med = float(np.median(kms))
    return {"prefill_ms": med, "prefill_TFLOPS": flops / (med * 1e-3) / 1e12,
            "pct_fp8_peak": 100 * flops / (med * 1e-3) / 1e12 / PEAK_FP8,
            "pipeline_ms": float(np.median(pipe)),
            "pipeline_TFLOPS": flops / (np.median(pipe) * 1e-3) / 1e12}


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


# ---------------------------------------------------------------------------
# rocprofv3 counter evidence: one probe per workload (a calibration copy and
# one launch of the workload's hot kernels), several counter passes, one
# summary per workload under profiles/
# ---------------------------------------------------------------------------
COUNTER_PASSES = {
    # MFMA pipe busy cycles / co-issue / instruction mix (8 SQ + 1 GRBM counters)
    "mfma": "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
            "SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES GRBM_GUI_ACTIVE",
    # MFMA operations executed per type (x512 = ops) and LDS use
    "mops": "SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
            "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_SALU GRBM_GUI_ACTIVE",
    # HBM-side bytes (in KiB per dispatch), one TCC-heavy counter per pass
    "fetch": "FETCH_SIZE GRBM_GUI_ACTIVE",
    "write": "WRITE_SIZE GRBM_GUI_ACTIVE",
}
SIMD_NUM = 1024   # 256 CUs x 4 SIMDs
XCD_NUM = 8       # GRBM_GUI_ACTIVE is reported summed over the 8 XCDs
PUBLISHED_GHZ = 2.4  # engine clock of the published peaks

# workload -> summary file, kernel-name patterns of its hot kernels, sources
COUNTER_WORKLOADS = {
    "c2": {"file": "counters_k_prefill_sage_varlen.md", "kernels": [r"k_prefill<128, 2, false, false, false>"],
           "title": "int8-QK / fp16-PV varlen prefill (SageAttention workload: B=8, lengths U{512..4096} seed "
                    "1002, causal, Hq=32, Hkv=8, D=128; 16-bit Q quantized in the kernel)",
           "sources": ("paged_kv_amd/csrc/prefill.hip", "paged_kv_amd/csrc/kcommon.h", "paged_kv_amd/csrc/launch.h")},
    "c5": {"file": "counters_k_prefill_fp8_long.md", "kernels": [r"k_prefill<128, 0, false, true, false>"],
           "title": "fp8 prefill, QK^T summed exactly on f16 MFMAs (long workload: B=1, S=32768, H=64, D=128, "
                    "causal, after RoPE + paged append + fp8 quantization)",
           "sources": ("paged_kv_amd/csrc/prefill.hip", "paged_kv_amd/csrc/kcommon.h", "paged_kv_amd/csrc/launch.h")},
    "c3": {"file": "counters_k_decode_paged_fp8.md", "kernels": [r"k_decode_split<128>", r"k_decode_merge<128>"],
           "title": "paged fp8 decode, split-KV + merge (B=64, kv lens U{1024..32768} seed 1003, page 16, "
                    "Hq=32, Hkv=8, D=128)",
           "sources": ("paged_kv_amd/csrc/decode.hip", "paged_kv_amd/csrc/kcommon.h", "paged_kv_amd/csrc/launch.h")},
    "c4": {"file": "counters_k_mla_sparse_decode.md", "kernels": [r"k_mla_split", r"k_mla_merge"],
           "title": "sparse MLA-absorb decode (B=32, 128 heads, 2048 selected 656-byte rows per query, "
                    "65536-token caches in 64-token blocks)",
           "sources": ("paged_kv_amd/csrc/mla.hip", "paged_kv_amd/csrc/mla.h", "paged_kv_amd/csrc/kcommon.h",
                       "paged_kv_amd/csrc/launch.h")},
}


def kernel_source_hash(sources) -> str:
    """Hash of the kernel sources with comments and blank lines removed (a
    comment edit does not change what the counters measured; the sources
    hold no string literal with a comment marker in it)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            line = line.split("//", 1)[0].rstrip()
            if line.strip():
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def _config2_flops():
    import gen
    return 4.0 * 128 * 32 * causal_pairs(gen.configs.config2_lengths())


def _algorithmic(wl):
    """(unit, algorithmic work of one launch of the workload's hot kernels)."""
    import gen
    if wl == "c2":
        return "flop", _config2_flops()
    if wl == "c5":
        return "flop", 4.0 * 128 * 64 * causal_pairs([32768])
    if wl == "c3":
        lens = gen.configs.config3_lengths().astype(np.int64)
        npages = (lens + 15) // 16
        return "byte", float(lens.sum() * 8 * 128 * 2 + 64 * 32 * 128 * 2 * 2 + npages.sum() * 4 + 65 * 4 * 2)
    if wl == "c4":
        return "byte", float(C4_BYTES)
    raise ValueError(wl)


C4_BYTES = 32 * 2048 * 656 + 32 * 128 * 576 * 2 + 32 * 128 * 512 * 2 + 32 * 2048 * 4 + 32 * 1024 * 4


def counter_probe(wl):
    """One calibration copy of CALIB_BYTES, then one launch of workload wl's
    hot kernels after its set-up (run under rocprofv3 --pmc, one pass per
    counter group)."""
    import torch
    import gen
    from tests.parity import to_dev
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    if wl == "c2":
        from paged_kv_amd.pipeline import SagePrefill
        x = gen.config2()
        p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["cu_seqlens"]),
                        int(x["seqlens"].max()), x["sm_scale"], causal=True)
        p.quantize()
        torch.cuda.synchronize()
        p.attend()
    elif wl == "c5":
        from paged_kv_amd.pipeline import AppendRopeFp8Prefill
        x = gen.config5()
        kc = torch.zeros((x["num_pages"], x["page_size"], 64, 128), dtype=torch.bfloat16, device="cuda")
        p = AppendRopeFp8Prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["cu_seqlens"]),
                                 to_dev(x["kv_len_before"]), 32768, to_dev(x["rope_cos_sin"]), kc, torch.zeros_like(kc),
                                 to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]), x["page_size"], x["sm_scale"])
        p.append()
        p.prefill.quantize()
        torch.cuda.synchronize()
        p.prefill.attend()
    elif wl == "c3":
        from paged_kv_amd.pipeline import PagedDecode
        x = gen.config3()
        p = PagedDecode(to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(x["k_scale"]),
                        to_dev(x["v_scale"]), to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]),
                        to_dev(x["kv_last_page_len"]), x["max_kv_len"], x["sm_scale"])
        torch.cuda.synchronize()
        p.run()
    elif wl == "c4":
        from paged_kv_amd.pipeline import SparseMlaDecode
        x = gen.config4()
        p = SparseMlaDecode(to_dev(x["q"]), to_dev(x["kv_cache"]), to_dev(x["block_table"]),
                            to_dev(x["kv_lens"]), to_dev(x["sparse_indices"]), x["sm_scale"])
        torch.cuda.synchronize()
        p.run()
    else:
        raise SystemExit(f"unknown workload {wl}")
    torch.cuda.synchronize()
    log(f"[bench] counter probe {wl} done")


def _counter_rows(d):
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return list(csv.DictReader(open(f[0])))


def _pass_values(d, patterns):
    """Counter values of one pass: (sum over the workload's hot-kernel
    dispatches, per-kernel values, calibration copy values, summed dispatch
    durations in ns)."""
    rows = _counter_rows(d)
    hot, per, copy = {}, {}, {}
    dur = {}
    for r in rows:
        name, cn, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
        if "copyBuffer" in name:
            copy[cn] = max(copy.get(cn, 0.0), v)
            continue
        for pat in patterns:
            if pat in name:
                per.setdefault(pat, {})[cn] = v          # the last dispatch of that kernel
                dur[pat] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    for pat, vals in per.items():
        for cn, v in vals.items():
            hot[cn] = hot.get(cn, 0.0) + v
    missing = [p for p in patterns if p not in per]
    if missing:
        raise SystemExit(f"{d}: no dispatch of {missing}")
    return hot, per, copy, float(sum(dur.values()))


def summarize_counters(wl, run_dir):
    """Write profiles/<file> for workload wl from the passes under run_dir
    (one subdirectory per pass, named as in COUNTER_PASSES, and cmds.txt with
    the commands that made them)."""
    cfg = COUNTER_WORKLOADS[wl]
    pats = cfg["kernels"]
    cmds = open(os.path.join(run_dir, "cmds.txt")).read().strip().splitlines()
    vals, per_kernel, copies, durs = {}, {}, {}, {}
    for pname in COUNTER_PASSES:
        d = os.path.join(run_dir, pname)
        if not os.path.isdir(d):
            continue
        hot, per, copy, dur = _pass_values(d, pats)
        vals.update({k: v for k, v in hot.items() if k != "GRBM_GUI_ACTIVE"})
        vals[f"GRBM_GUI_ACTIVE[{pname}]"] = hot.get("GRBM_GUI_ACTIVE", 0.0)
        for pat, pv in per.items():
            per_kernel.setdefault(pat, {}).update({k: v for k, v in pv.items() if k != "GRBM_GUI_ACTIVE"})
        copies[pname] = copy
        durs[pname] = dur
    unit, work = _algorithmic(wl)
    lines = [f"# rocprofv3 counters: {cfg['title']}", "",
             "Kernels: " + ", ".join(f"`{p}`" for p in pats) + " (one launch each, counters summed over them).", "",
             "Commands (repository root on the GPU host; `cd /tmp && export TMPDIR=/tmp` first, R = the root):", ""]
    lines += [f"    {c}" for c in cmds]
    lines += ["", "| counter | " + " | ".join(f"`{p}`" for p in pats) + " | total |",
              "|---|" + "---|" * (len(pats) + 1)]
    for cn in sorted(k for k in vals if not k.startswith("GRBM")):
        lines.append(f"| {cn} | " + " | ".join(f"{per_kernel[p].get(cn, float('nan')):.6g}" for p in pats)
                     + f" | {vals[cn]:.6g} |")
    for k in sorted(k for k in vals if k.startswith("GRBM")):
        lines.append(f"| {k} | | {vals[k]:.6g} |")
    derived = {}
    lines += ["", "Derived (per launch):", ""]
    if "mfma" in durs:
        grbm = vals["GRBM_GUI_ACTIVE[mfma]"] / XCD_NUM          # cycles of one XCD
        util = 100.0 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (grbm * SIMD_NUM)
        # the same busy cycles over the dispatch time at the published clock
        # (a lower bound: the clock under load is at most that)
        util_t = 100.0 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMD_NUM * durs["mfma"] * PUBLISHED_GHZ)
        clock = grbm / max(durs["mfma"], 1.0)
        coexec = 100.0 * vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(vals["SQ_VALU_MFMA_BUSY_CYCLES"], 1.0)
        # GRBM_GUI_ACTIVE runs ahead of the dispatch for short launches under
        # counter collection (an implied clock above the published one): then
        # the dispatch-time figure is the one to use
        derived["mfma_util_pct"] = util if clock <= PUBLISHED_GHZ else util_t
        lines += [f"- MFMA pipe busy (rocprof's MfmaUtil: sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE of one XCD "
                  f"x {SIMD_NUM} SIMDs)): **{util:.1f}%**"
                  + ("" if clock <= PUBLISHED_GHZ else
                     f" -- not usable here: the implied clock ({clock:.2f} GHz) is above the published "
                     f"{PUBLISHED_GHZ} GHz, i.e. GRBM_GUI_ACTIVE counted well beyond the dispatch"),
                  f"- MFMA pipe busy over the summed dispatch time ({durs['mfma'] / 1e3:.1f} us) at {PUBLISHED_GHZ} GHz: "
                  f"**{util_t:.1f}%** (a lower bound)",
                  f"- cycles with a VALU instruction issued beside a busy MFMA pipe: {coexec:.1f}% of the MFMA busy cycles",
                  f"- VALU instructions per MFMA instruction: {vals['SQ_INSTS_VALU'] / max(vals['SQ_INSTS_MFMA'], 1):.2f} "
                  f"(transcendental fp32: {vals['SQ_INSTS_VALU_TRANS_F32'] / max(vals['SQ_INSTS_MFMA'], 1):.2f})",
                  f"- engine clock under the kernel: {grbm / max(durs['mfma'], 1.0):.3f} GHz (GRBM_GUI_ACTIVE of one XCD "
                  f"/ dispatch time {durs['mfma'] / 1e3:.1f} us)"]
    if "mops" in durs:
        ops = {t: 512.0 * vals.get(f"SQ_INSTS_VALU_MFMA_MOPS_{t}", 0.0) for t in ("I8", "F8", "F16", "BF16")}
        tot = sum(ops.values())
        derived["mfma_ops"] = tot
        lines += ["- MFMA operations executed: " + ", ".join(f"{t} {v:.4g}" for t, v in ops.items() if v)
                  + f"; total {tot:.4g}"]
        if unit == "flop":
            lines += [f"- algorithmic flop of the launch {work:.4g}: executed / algorithmic = {tot / work:.3f} "
                      "(tiles crossing the causal diagonal or a sequence end are computed whole)"]
    if "fetch" in durs and "write" in durs:
        fcal = (CALIB_BYTES / 1024.0) / copies["fetch"]["FETCH_SIZE"]
        wcal = (CALIB_BYTES / 1024.0) / copies["write"]["WRITE_SIZE"]
        fb = vals["FETCH_SIZE"] * fcal * 1024.0
        wb = vals["WRITE_SIZE"] * wcal * 1024.0
        derived["traffic"] = fb + wb
        lines += [f"- HBM-side traffic: FETCH_SIZE {vals['FETCH_SIZE']:.0f} KiB x {fcal:.4f} + WRITE_SIZE "
                  f"{vals['WRITE_SIZE']:.0f} KiB x {wcal:.4f} = {fb:.4g} + {wb:.4g} = **{fb + wb:.4g} bytes** "
                  f"(factors: {CALIB_BYTES >> 20} MiB device copy, {CALIB_BYTES / 1024:.0f} KiB each way, read "
                  f"{copies['fetch']['FETCH_SIZE']:.0f} KiB fetched and {copies['write']['WRITE_SIZE']:.0f} KiB written)"]
        if unit == "byte":
            lines += [f"- algorithmic bytes {work:.4g}: traffic / algorithmic = {(fb + wb) / work:.3f}",
                      f"- at the dispatch time of the fetch pass ({durs['fetch'] / 1e3:.1f} us, caches as the probe left "
                      f"them): {work / durs['fetch']:.1f} GB/s algorithmic, {(fb + wb) / durs['fetch']:.1f} GB/s measured"]
    lines += ["", "Machine-readable:", ""]
    if "traffic" in derived:
        lines.append(f"traffic_bytes_per_launch: {derived['traffic']:.6g}")
    if "mfma_util_pct" in derived:
        lines.append(f"mfma_util_pct: {derived['mfma_util_pct']:.4g}")
    if "mfma_ops" in derived:
        lines.append(f"mfma_ops_per_launch: {derived['mfma_ops']:.6g}")
    lines += [f"kernel_source_hash: {kernel_source_hash(cfg['sources'])}", ""]
    out = os.path.join(ROOT, "profiles", cfg["file"])
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps({"file": out, **derived}))


def stored_counters(wl):
    """Machine-readable figures of workload wl's counter summary, or {} when
    the kernel sources changed since the counters were taken."""
    cfg = COUNTER_WORKLOADS[wl]
    try:
        txt = open(os.path.join(ROOT, "profiles", cfg["file"])).read()
    except OSError:
        return {}
    vals = dict(l.split(": ", 1) for l in txt.splitlines()
                if l.startswith(("traffic_bytes_per_launch", "kernel_source_hash", "mfma_util_pct", "mfma_ops_per_launch")))
    if vals.get("kernel_source_hash") != kernel_source_hash(cfg["sources"]):
        return {}
    return {k: float(v) for k, v in vals.items() if k != "kernel_source_hash"}


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
    ap.add_argument("--extra", default="c3,c5,c4,paged,paged_fp8",
                    help="comma list of extra workloads (c3,c4,c5,paged,paged_fp8) or ''")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counter-probe", choices=sorted(COUNTER_WORKLOADS),
                    help="run the calibration copy and one launch of a workload's hot kernels (for rocprofv3 --pmc)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("WORKLOAD", "RUN_DIR"),
                    help="write profiles/counters_*.md from the counter passes under RUN_DIR")
    ap.add_argument("--list-counter-passes", action="store_true",
                    help="print the counter groups of the passes, one per line (name: counters)")
    a = ap.parse_args()
    if a.summarize_counters:
        summarize_counters(*a.summarize_counters)
        return
    if a.list_counter_passes:
        for k, v in COUNTER_PASSES.items():
            print(f"{k}: {v}")
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    import paged_kv_amd
    paged_kv_amd.lib()
    if a.counter_probe:
        counter_probe(a.counter_probe)
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
                         ("paged", bench_paged_prefill, 10), ("paged_fp8", bench_paged_prefill_fp8, 10)):
        if name not in a.extra.split(","):
            continue
        log(f"[bench] {name}")
        try:
            kw = {} if name == "paged_fp8" else {"cpu": not a.no_cpu_baseline}
            extra[{"c3": "config3_decode", "c5": "config5_long_prefill", "c4": "config4_sparse_mla",
                   "paged": "chunked_prefill_paged", "paged_fp8": "chunked_prefill_paged_fp8"}[name]] = \
                fn(it, **kw)
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
                     "frac": k_tflops / peak_mixed, "traffic": stored_counters("c2").get("traffic_bytes_per_launch"),
                     "mfma_util_pct": stored_counters("c2").get("mfma_util_pct"),
                     "kernel": "k_prefill<128, int8 QK, fp16 V>",
                     "per_launch_flop": r2["flops"], "avg_launch_ms": r2["kernel_ms"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
