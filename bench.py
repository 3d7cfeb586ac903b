#!/usr/bin/env python3
"""Benchmark of the INT8-QK paged-attention hot path on one MI355X.

Headline workload: Qwen3.5-27B-shaped decode (24 query heads over 4 KV heads,
head_dim 256, 32768 cached tokens, INT8 K with per-token scales, bf16 V).
One step = qa_paged_decode_step: quantize the new query token, write the
new token's K/V into the paged cache and run split-K paged decode attention
(one kernel), then merge the splits (a second kernel). The metric is
algorithmic bytes per second.

Steps rotate over several independently allocated KV pools, so together
they exceed the 256 MB Infinity Cache and each step streams its cache from
HBM.

Prints one JSON line. Extra keys: the roofline of the split kernel (HIP
events around batches of back-to-back launches of the step's first phase,
after the timed step loop), the oracle's CPU
throughput on a bounded sample, and throughput of the prefill and dense
paths on their own workloads.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# MI355X published dense matrix peaks (no sparsity)
INT8_PEAK_TOPS = 5000.0
FP16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0


def decode_bytes(spec) -> dict:
    """Algorithmic bytes of one decode step (one new token per sequence):
    the cached K codes, K scales and V (and V scales) of every context token,
    the block table, the bf16 query, the new token's bf16 K/V and its slot,
    the new token's cache row (written), and the fp32 output."""
    d, Hq, Hkv = spec.head_dim, spec.num_q_heads, spec.num_kv_heads
    tok = sum(spec.context_lens)
    v_elem = 1 if spec.v_int8 else 2
    row = d + 4 + d * v_elem + (4 if spec.v_int8 else 0)      # one (token, KV head) in the cache
    hist = (tok * Hkv * row                                     # K, sK, V (, sV)
            + sum(spec.blocks_per_seq) * 4                       # the block-table entries in use
            + spec.num_seqs * Hq * d * 4)                       # fp32 output
    step = (hist + spec.num_seqs * Hq * 2 * d                   # bf16 query
            + spec.num_seqs * (Hkv * (4 * d + row) + 8))        # new K/V in, its cache row out, slot
    return {"history": hist, "step": step}


def flash_ops(q_lens, ctx_lens, Hq, d, causal=True):
    """QK (INT8) and PV (fp16) operations of prefill/dense: 2*d each per
    visible (query, key) pair."""
    pairs = 0
    for tq, c in zip(q_lens, ctx_lens):
        if causal:
            off = c - tq
            pairs += sum(min(c, off + i + 1) for i in range(tq))
        else:
            pairs += tq * c
    pairs *= Hq
    return 2 * d * pairs, 2 * d * pairs


def dev_bits(torch, bits: np.ndarray, dtype: str = "bf16"):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def gpu_cache(torch, qa, inp):
    spec = inp.spec
    kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, spec.num_kv_heads, spec.head_dim,
                                       torch.int8 if spec.v_int8 else torch.bfloat16)
    qa.write_kv_cache(dev_bits(torch, inp.k), dev_bits(torch, inp.v), torch.from_numpy(inp.slot_mapping).cuda(),
                      kc, ks, vc, vs)
    return kc, ks, vc, vs


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_qwen27b_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_attention_quantize_amd", "csrc", f)
                  for f in ("decode.hip", "common.h", "internal.h")]


def kernel_source_digest() -> str:
    """sha256 over what the decode kernel is built from: decode.hip,
    common.h and the DecodeArgs declaration of internal.h (the header's
    other structs belong to other kernels)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            text = fh.read()
        if f.endswith("internal.h"):
            i = text.index(b"struct DecodeArgs {")
            text = text[i:text.index(b"};", i) + 2]
        h.update(text)
    return h.hexdigest()


def decode_traffic():
    """HBM bytes per k_decode launch from the committed counter summary, or
    None when the summary is missing or the kernel sources have changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.split(":", 1) for line in fh if line.startswith(("traffic_bytes_per_launch:",
                                                                            "kernel_source_sha256:")))
    except OSError:
        return None
    if kv.get("kernel_source_sha256", "").strip() != kernel_source_digest():
        return None
    return int(kv["traffic_bytes_per_launch"].strip())


def _mk_stream_events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def run_decode(args, torch, qa, W):
    from workloads import qwen27b_decode, paged_inputs
    spec = qwen27b_decode(args.context)
    inp = paged_inputs(spec)
    dev = torch.device("cuda:0")
    d, Hq, Hkv = spec.head_dim, spec.num_q_heads, spec.num_kv_heads
    # pool 0: write every token; pools 1..R-1: device copies at other addresses
    slots = torch.from_numpy(inp.slot_mapping).to(dev)
    kb, vb = dev_bits(torch, inp.k), dev_bits(torch, inp.v)
    pools = []
    for r in range(args.pools):
        kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, Hkv, d, torch.bfloat16, zero=False)
        if r == 0:
            qa.write_kv_cache(kb, vb, slots, kc, ks, vc, vs)
        else:
            kc.copy_(pools[0][0]); ks.copy_(pools[0][1]); vc.copy_(pools[0][2])
        pools.append((kc, ks, vc, vs))
    # the step's new token is the last one of the context
    k_new, v_new = kb[-1:].contiguous(), vb[-1:].contiguous()
    slot_new = slots[-1:].contiguous()
    del kb, vb
    q = dev_bits(torch, inp.q)
    tables = torch.from_numpy(inp.block_tables).to(dev)
    lens = torch.from_numpy(inp.context_lens).to(dev)
    p = qa.decode_params(spec.num_seqs, Hq, Hkv, d, spec.max_blocks_per_seq, spec.num_blocks,
                         num_splits=args.splits)
    splits = qa.decode_num_splits(p)
    ws = qa.decode_workspace(p, dev)
    out = torch.empty((spec.num_seqs, Hq, d), dtype=torch.float32, device=dev)
    import ctypes
    L = qa.lib

    def step(i):
        # one call: quantize the query, write the new token's K/V, attend
        kc, ks, vc, vs = pools[i % len(pools)]
        qa._check(L.qa_paged_decode_step(
            ctypes.byref(p), qa._ptr(q), Hq * d, d, qa._ptr(k_new), qa._ptr(v_new), Hkv * d, d, qa.QA_DT_BF16,
            qa._ptr(slot_new), qa._ptr(kc), qa._ptr(ks), qa._ptr(vc), None, qa._ptr(tables), qa._ptr(lens),
            qa._ptr(ws), ws.numel(), qa._ptr(out), qa._stream()))

    def partials(i):
        kc, ks, vc, vs = pools[i % len(pools)]
        qa._check(L.qa_paged_decode_step_partials(
            ctypes.byref(p), qa._ptr(q), Hq * d, d, qa._ptr(k_new), qa._ptr(v_new), Hkv * d, d, qa.QA_DT_BF16,
            qa._ptr(slot_new), qa._ptr(kc), qa._ptr(ks), qa._ptr(vc), None, qa._ptr(tables), qa._ptr(lens),
            qa._ptr(ws), ws.numel(), qa._ptr(out), qa._stream()))

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(K):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K

    # k_decode alone: batches of back-to-back launches of the step's first
    # phase (pools rotated as in the step loop) between two HIP events on
    # torch's current stream, which the library launches on. The host
    # enqueues a launch faster than the kernel runs, so the events see the
    # kernels and the gaps between them, not the host.
    def batches(fn, n_batches, per):
        evs = _mk_stream_events(torch, n_batches)
        torch.cuda.synchronize()
        for b in range(n_batches):
            evs[b][0].record()
            for j in range(per):
                fn(b * per + j)
            evs[b][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(e) / per for a, e in evs]

    per = 10
    kern_ms = batches(partials, max(1, K // per), per)

    rope_ms = None
    if not args.no_extras:
        # the same step with rotary embedding in the split kernel (a quarter
        # of the head rotated, half pairing; positions = context - 1)
        from workloads import rope_table
        tab = torch.from_numpy(rope_table(args.context, 64)).to(dev)
        pos = (lens - 1).to(torch.int64)
        rp = qa.RopeParams(qa._ptr(pos), qa._ptr(tab), 64, 1)

        def step_rope(i):
            kc, ks, vc, vs = pools[i % len(pools)]
            qa._check(L.qa_paged_decode_step_rope(
                ctypes.byref(rp), ctypes.byref(p), qa._ptr(q), Hq * d, d, qa._ptr(k_new), qa._ptr(v_new), Hkv * d,
                d, qa.QA_DT_BF16, qa._ptr(slot_new), qa._ptr(kc), qa._ptr(ks), qa._ptr(vc), None, qa._ptr(tables),
                qa._ptr(lens), qa._ptr(ws), ws.numel(), qa._ptr(out), qa._stream()))
        for i in range(W):
            step_rope(i)
        torch.cuda.synchronize()
        t0.record()
        for i in range(K):
            step_rope(i)
        t1.record()
        torch.cuda.synchronize()
        rope_ms = t0.elapsed_time(t1) / K

    step(0)                            # the output checked against the oracle (cpu_baseline leg)
    torch.cuda.synchronize()
    out_host = out.cpu().numpy()
    nbytes = decode_bytes(spec)
    return spec, {
        "ms_per_step": ms_step,
        "value": nbytes["step"] / (ms_step * 1e-3) / 1e9,
        "kernel_ms": float(np.mean(kern_ms)),
        "kernel_ms_p10_p90": [float(np.percentile(kern_ms, 10)), float(np.percentile(kern_ms, 90))],
        "step_bytes": nbytes["step"],
        "splits": splits,
        "rope_ms_per_step": rope_ms,
        "inp": inp,
        "out": out_host,
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, inp, budget_s, gpu_out=None):
    """The oracle (C++17, oracle/), untuned, on the decode workload: quantize
    the query and run unsplit paged decode over the cache the oracle writes
    itself, once with one OpenMP thread per host cpu (its parallel units are
    the (sequence, query head) pairs) and once on one thread. Also reports
    the GPU step's output against the oracle's (same inputs)."""
    import oracle
    caches = oracle.write_kv_cache(inp.k, inp.v, "bf16", inp.slot_mapping, spec.num_blocks)
    nproc = len(os.sched_getaffinity(0))
    units = spec.num_seqs * spec.num_q_heads

    def run(threads, budget):
        oracle.set_num_threads(threads)
        n, t_total, out = 0, 0.0, None
        while t_total < budget or n == 0:
            t = time.perf_counter()
            q8, qs = oracle.quantize_q(inp.q)
            out = oracle.paged_decode(q8, qs, caches, inp.block_tables, inp.context_lens, spec.num_kv_heads)
            t_total += time.perf_counter() - t
            n += 1
            if n >= 1000:
                break
        return n, t_total, out

    n, t_total, ref = run(nproc, 0.6 * budget_s)
    n1, t1, _ = run(1, 0.4 * budget_s)
    oracle.set_num_threads(nproc)
    by = decode_bytes(spec)["step"]
    used = min(nproc, units)
    model = _cpu_model()
    res = {"value": by * n / t_total / 1e9, "unit": "GB/s", "cores": used, "kind": "oracle",
           "sample": f"{n} full decode steps (C++ oracle: quantize_q + unsplit paged decode in fp64) of the "
                     f"{spec.context_lens[0]}-token workload in {t_total:.1f} s with {used} OpenMP threads "
                     f"(one per (sequence, query head) unit, {nproc} host cpus: {model})",
           "one_thread": {"value": by * n1 / t1 / 1e9, "unit": "GB/s", "steps": n1, "seconds": round(t1, 2)},
           "host": {"nproc": nproc, "cpu_model": model}}
    if gpu_out is not None:
        want = np.asarray(ref, np.float64).reshape(gpu_out.shape)
        got = gpu_out.astype(np.float64)
        res["gpu_parity"] = {"rel_l2": float(np.linalg.norm(got - want) / np.linalg.norm(want)),
                             "max_abs": float(np.max(np.abs(got - want))),
                             "bar": "rel L2 <= 1e-3, max abs <= 2e-3 (fp32 output)"}
        # the method's own error: the GPU output against textbook fp64
        # attention of the unquantized bf16 query, keys and values
        G = spec.num_q_heads // spec.num_kv_heads
        q = oracle.widen(inp.q, "bf16").astype(np.float64)[0]                  # [Hq, d]
        k = oracle.widen(inp.k, "bf16").astype(np.float64)                      # [ctx, Hkv, d]
        v = oracle.widen(inp.v, "bf16").astype(np.float64)
        sc = 1.0 / np.sqrt(spec.head_dim)
        exact = np.stack([oracle.attention_fp64(q[h:h + 1], k[:, h // G], v[:, h // G], sc)[0]
                          for h in range(spec.num_q_heads)])
        g0 = got.reshape(exact.shape)
        res["gpu_vs_unquantized_fp64"] = {"rel_l2": float(np.linalg.norm(g0 - exact) / np.linalg.norm(exact)),
                                          "max_abs": float(np.max(np.abs(g0 - exact)))}
    return res


def run_decode_mt(torch, qa, context, T, pools, reps=50):
    """Multi-token decode on the Qwen3.5-27B shape: T query tokens per step
    (24 query heads x T in the 16 matrix columns of each KV head), the cache
    already holding them; pools rotated as in the decode bench. Bytes per
    call: the cache rows of every context token (as in decode), the block
    table, the INT8 query codes and scales, and the fp32 output."""
    from workloads import PagedSpec, paged_inputs
    spec = PagedSpec("qwen27b_decode_mt", 2, 1, 24, 4, 256, [context], [T], k_bias_std=2.0)
    inp = paged_inputs(spec)
    kc, ks, vc, vs = gpu_cache(torch, qa, inp)
    caches = [(kc, ks, vc, vs)]
    for _ in range(pools - 1):
        caches.append((kc.clone(), ks.clone(), vc.clone(), vs))
    q8, qs = qa.quantize_q(dev_bits(torch, inp.q))
    S, Hq, d = 1, 24, 256
    q8, qs = q8.view(S, T, Hq, d), qs.view(S, T, Hq)
    tables = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    out = torch.empty((S, T, Hq, d), device="cuda")
    f = lambda i: qa.paged_attention_decode_mt(q8, qs, *caches[i % pools], tables, lens, out=out)
    for i in range(10):
        f(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(reps):
        f(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    row = d + 4 + 2 * d
    nbytes = context * 4 * row + spec.max_blocks_per_seq * 4 + T * Hq * (d + 4) + T * Hq * d * 4
    return {"workload": f"qwen27b decode, {T} query tokens per step, context {context} "
                        f"(G x T = {6 * T} of 16 matrix columns)",
            "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes": nbytes, "note": "one call: split kernel + combine (query already quantized)"}


def run_prefill(torch, qa, reps, pv_fp8=False, v_ws=False):
    """The chunked prefill workload; with pv_fp8 the FP8 P.V call (its two
    V passes included in the time); with v_ws the call that converts V once
    into a workspace (that pass included)."""
    from workloads import chunked_prefill, paged_inputs
    spec = chunked_prefill()
    inp = paged_inputs(spec)
    kc, ks, vc, vs = gpu_cache(torch, qa, inp)
    q8, qs = qa.quantize_q(dev_bits(torch, inp.q))
    cu = torch.from_numpy(inp.cu_seqlens_q).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    tables = torch.from_numpy(inp.block_tables).cuda()
    out = torch.empty((spec.total_q, spec.num_q_heads, spec.head_dim), device="cuda")
    if pv_fp8:
        ws = qa.chunked_prefill_fp8pv_workspace(qa.prefill_params(q8, lens, kc, vc, tables, spec.query_lens[0]))
        f = lambda: qa.chunked_prefill_attention_fp8pv(q8, qs, cu, lens, kc, ks, vc, vs, tables, spec.query_lens[0],
                                                       workspace=ws, out=out)
    elif v_ws:
        ws = qa.chunked_prefill_ws_workspace(qa.prefill_params(q8, lens, kc, vc, tables, spec.query_lens[0]))
        f = lambda: qa.chunked_prefill_attention_ws(q8, qs, cu, lens, kc, ks, vc, vs, tables, spec.query_lens[0],
                                                    workspace=ws, out=out)
    else:
        f = lambda: qa.chunked_prefill_attention(q8, qs, cu, lens, kc, ks, vc, vs, tables, spec.query_lens[0],
                                                 out=out)
    for _ in range(3):
        f()
    evs = _mk_stream_events(torch, reps)
    for a, b in evs:
        a.record(); f(); b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    qk, pv = flash_ops(spec.query_lens, spec.context_lens, spec.num_q_heads, spec.head_dim)
    tops = (qk + pv) / (ms * 1e-3) / 1e12
    mixed = (qk / (INT8_PEAK_TOPS * 1e12) + pv / ((FP8_PEAK_TFLOPS if pv_fp8 else FP16_PEAK_TFLOPS) * 1e12)) / (ms * 1e-3)
    return {"workload": "chunked_prefill 2048 new tokens on 16384 history, 24/4 heads, d256"
                        + (", FP8 E4M3 P.V (V scale and E4M3 passes included)" if pv_fp8 else "")
                        + (", V converted once into a workspace (that pass included)" if v_ws else ""),
            "ms": ms, "TOPS": tops, "frac_int8_peak": tops / INT8_PEAK_TOPS, "frac_mixed_roofline": mixed,
            "_ops": (qk, pv, "fp8" if pv_fp8 else "f16")}


def run_dense(torch, qa, reps, causal, options=False, pv_fp8=False):
    """The dense workload; with options, through the options call in the HND
    layout with smooth_v and the LSE output; with pv_fp8, the options call
    (NHD) with the P.V product in FP8."""
    from workloads import dense_sage, dense_inputs
    spec = dense_sage()
    inp = dense_inputs(spec)
    q, k, v = (dev_bits(torch, x, "f16") for x in (inp.q, inp.k, inp.v))
    p = qa.dense_params(q, k, True, causal)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    if options:
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
        o = qa.DenseOptions(qa.QA_LAYOUT_HND, 1)
        ws = torch.empty(qa.lib.qa_dense_sage_ex_workspace_size(ctypes.byref(p), ctypes.byref(o)),
                         dtype=torch.uint8, device="cuda")
        out = out.transpose(1, 2).contiguous()
        lse = torch.empty((spec.batch, spec.num_q_heads, spec.seq_q), dtype=torch.float32, device="cuda")
        f = lambda: qa.dense_sage_attention_ex(q, k, v, "HND", is_causal=causal, smooth_v=True, return_lse=True,
                                               workspace=ws, out=out, lse=lse)
    elif pv_fp8:
        o = qa.DenseOptions(qa.QA_LAYOUT_NHD, 0, 1)
        ws = torch.empty(qa.lib.qa_dense_sage_ex_workspace_size(ctypes.byref(p), ctypes.byref(o)),
                         dtype=torch.uint8, device="cuda")
        f = lambda: qa.dense_sage_attention_ex(q, k, v, is_causal=causal, pv_fp8=True, workspace=ws, out=out)
    else:
        ws = qa.dense_sage_workspace(p)
        f = lambda: qa.dense_sage_attention(q, k, v, is_causal=causal, workspace=ws, out=out)
    for _ in range(3):
        f()
    evs = _mk_stream_events(torch, reps)
    for a, b in evs:
        a.record(); f(); b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    B, H, N, d = spec.batch, spec.num_q_heads, spec.seq_q, spec.head_dim
    qk, pv = flash_ops([N] * B, [N] * B, H, d, causal)
    tops = (qk + pv) / (ms * 1e-3) / 1e12
    pv_peak = FP8_PEAK_TFLOPS if pv_fp8 else FP16_PEAK_TFLOPS
    mixed = (qk / (INT8_PEAK_TOPS * 1e12) + pv / (pv_peak * 1e12)) / (ms * 1e-3)
    return {"workload": f"dense_sage B2 H32 N8192 d128 {'causal' if causal else 'non-causal'} "
                        "(full chain: smooth_k + per-block quantization + attention"
                        + (", HND, smooth_v, LSE output)" if options else ", FP8 E4M3 P.V)" if pv_fp8 else ")"),
            "ms": ms, "TOPS": tops, "frac_int8_peak": tops / INT8_PEAK_TOPS, "frac_mixed_roofline": mixed,
            "_ops": (qk, pv, "fp8" if pv_fp8 else "f16")}


def _timed_ms(torch, fn, reps, warm=3):
    """Median of `reps` launches of fn between HIP events on torch's current
    stream (the stream the library launches on)."""
    for _ in range(warm):
        fn(0)
    evs = _mk_stream_events(torch, reps)
    for i, (a, b) in enumerate(evs):
        a.record(); fn(i); b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def _step_call(torch, qa, spec, inp, pools_n, splits):
    """A decode-step closure over `pools_n` separately allocated copies of the
    cache (the new token of every sequence is its last one)."""
    dev = torch.device("cuda:0")
    d, Hq, Hkv = spec.head_dim, spec.num_q_heads, spec.num_kv_heads
    v_dt = torch.int8 if spec.v_int8 else torch.bfloat16
    slots = torch.from_numpy(inp.slot_mapping).to(dev)
    kb, vb = dev_bits(torch, inp.k), dev_bits(torch, inp.v)
    pools = []
    for r in range(pools_n):
        kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, Hkv, d, v_dt, zero=False)
        if r == 0:
            qa.write_kv_cache(kb, vb, slots, kc, ks, vc, vs)
        else:
            kc.copy_(pools[0][0]); ks.copy_(pools[0][1]); vc.copy_(pools[0][2])
            if vs is not None:
                vs.copy_(pools[0][3])
        pools.append((kc, ks, vc, vs))
    last = torch.from_numpy(inp.cu_seqlens_kv[1:] - 1).to(dev)          # each sequence's last token
    k_new, v_new, slot_new = kb[last].contiguous(), vb[last].contiguous(), slots[last].contiguous()
    del kb, vb
    q = dev_bits(torch, inp.q)
    tables = torch.from_numpy(inp.block_tables).to(dev)
    lens = torch.from_numpy(inp.context_lens).to(dev)
    p = qa.decode_params(spec.num_seqs, Hq, Hkv, d, spec.max_blocks_per_seq, spec.num_blocks,
                         v_int8=spec.v_int8, num_splits=splits)
    ws = qa.decode_workspace(p, dev)
    out = torch.empty((spec.num_seqs, Hq, d), dtype=torch.float32, device=dev)
    L = qa.lib

    def step(i, fn=None):
        kc, ks, vc, vs = pools[i % len(pools)]
        qa._check((fn or L.qa_paged_decode_step)(
            ctypes.byref(p), qa._ptr(q), Hq * d, d, qa._ptr(k_new), qa._ptr(v_new), Hkv * d, d, qa.QA_DT_BF16,
            qa._ptr(slot_new), qa._ptr(kc), qa._ptr(ks), qa._ptr(vc), qa._ptr(vs), qa._ptr(tables), qa._ptr(lens),
            qa._ptr(ws), ws.numel(), qa._ptr(out), qa._stream()))
    return step, p, out


def run_decode_batched(torch, qa, reps=30, pools=2, splits=None):
    """Batched split-K decode: 32 sequences with contexts uniform on [1024,
    32768] (seeded), 24/4 heads, d 256, INT8 K and INT8 V with per-token
    scales, 8 splits per sequence. One step = qa_paged_decode_step (query
    quantized inside the split kernel, new token written) + the combine.
    Two cache copies (1.1 GB each) alternate, more than the 256 MB
    Infinity Cache holds. Bytes as decode_bytes: the exact sum over the
    seeded contexts."""
    from workloads import batched_splitk_decode, paged_inputs
    spec = batched_splitk_decode()
    inp = paged_inputs(spec)
    S = splits if splits is not None else spec.num_splits
    step, p, _ = _step_call(torch, qa, spec, inp, pools, S)
    S_run = qa.lib.qa_paged_decode_num_splits(ctypes.byref(p))
    ms = _timed_ms(torch, step, reps)
    part = _timed_ms(torch, lambda i: step(i, qa.lib.qa_paged_decode_step_partials), reps)
    by = decode_bytes(spec)["step"]
    how = f"{S_run} splits" + (" (library choice)" if S == 0 else "")
    return {"workload": f"batched split-K decode: 32 sequences, contexts U[1024, 32768] (sum {sum(spec.context_lens)}), "
                        f"24/4 heads, d256, INT8 K + INT8 V, {how}; step = fused quantize/write/split kernel + combine",
            "ms": ms, "GBps": by / (ms * 1e-3) / 1e9, "frac_hbm_peak": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes": by, "split_kernel_ms": part, "split_kernel_frac_hbm_peak": by / (part * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kv_pools": pools}


def run_decode_tiny(torch, qa, reps=200):
    """The tiny decode (6/1 heads, d 64, context 256): latency of one step."""
    from workloads import tiny_decode, paged_inputs
    spec = tiny_decode()
    inp = paged_inputs(spec)
    step, p, _ = _step_call(torch, qa, spec, inp, 1, 0)
    # back-to-back steps between two events (one step alone would time the
    # host's launch latency, not the GPU)
    for i in range(10):
        step(i)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(reps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    by = decode_bytes(spec)["step"]
    return {"workload": "tiny decode: 1 sequence, 6/1 heads, d64, context 256, bf16 V; one step "
                        f"({qa.decode_num_splits(p)} splits)", "us": ms * 1e3, "bytes": by}


def _batched_us(torch, fn, batch=20, reps=9, warm=3):
    """Per-launch time of fn in microseconds: the median over `reps` batches
    of `batch` back-to-back launches between HIP events on torch's current
    stream (the stream the library launches on), so that kernels shorter than
    the host's call overhead are still timed by the GPU's clock."""
    for _ in range(warm):
        fn()
    evs = _mk_stream_events(torch, reps)
    for a, b in evs:
        a.record()
        for _ in range(batch):
            fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3 / batch


def run_producers(torch, qa, reps=50):
    """quantize_q and write_kv_cache on their own, on the chunked-prefill
    shapes: 2048 query tokens x 24 heads x 256 (bf16 in, INT8 codes + fp32
    scales out) and 2048 new tokens x 4 KV heads written into the paged cache
    (K quantized, bf16 V copied). Bytes read + written."""
    from workloads import chunked_prefill, paged_inputs
    spec = chunked_prefill()
    inp = paged_inputs(spec)
    T, Hq, Hkv, d = spec.total_q, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    q = dev_bits(torch, inp.q)
    q8 = torch.empty((T, Hq, d), dtype=torch.int8, device="cuda")
    qs = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    L = qa.lib
    # the C-ABI calls with their arguments marshalled once (host cost per
    # launch well under the kernels' durations)
    stream = qa._stream()
    qa_args = (qa._ptr(q), qa.QA_DT_BF16, T, Hq, d, Hq * d, d, qa._ptr(q8), qa._ptr(qs), stream)
    fq = lambda: qa._check(L.qa_quantize_q(*qa_args))
    us_q = _batched_us(torch, fq)
    bq = T * Hq * (2 * d + d + 4)
    kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, Hkv, d, torch.bfloat16)
    kb = dev_bits(torch, inp.k[-T:])
    vb = dev_bits(torch, inp.v[-T:])
    slots = torch.from_numpy(inp.slot_mapping[-T:].copy()).cuda()
    qa.write_kv_cache(kb, vb, slots, kc, ks, vc, vs)   # argument checks of the binding, once
    kv_args = (qa._ptr(kb), qa._ptr(vb), qa.QA_DT_BF16, T, Hkv, d, kb.stride(0), kb.stride(1), qa._ptr(slots),
               kc.shape[0], 16, qa._ptr(kc), qa._ptr(ks), qa._ptr(vc), qa.QA_DT_BF16, None, stream)
    fw = lambda: qa._check(L.qa_write_kv_cache(*kv_args))
    us_w = _batched_us(torch, fw)
    bw = T * Hkv * (2 * d + 2 * d + d + 4 + 2 * d) + 8 * T
    # a plain device copy moving the same bytes (half read, half written):
    # the practical floor of a read + write stream of this size
    def copy_us(nbytes):
        src = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        return _batched_us(torch, lambda: dst.copy_(src))
    cq, cw = copy_us(bq), copy_us(bw)
    ms_q, ms_w = us_q * 1e-3, us_w * 1e-3
    return {"quantize_q": {"workload": f"{T} tokens x {Hq} heads x {d}, bf16 -> INT8 + fp32 scale",
                           "us": ms_q * 1e3, "GBps": bq / (ms_q * 1e-3) / 1e9,
                           "frac_hbm_peak": bq / (ms_q * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": bq,
                           "copy_same_bytes_us": cq},
            "write_kv_cache": {"workload": f"{T} tokens x {Hkv} KV heads x {d}: K quantized into the paged INT8 "
                                           "layout with per-token scales, bf16 V copied",
                               "us": ms_w * 1e3, "GBps": bw / (ms_w * 1e-3) / 1e9,
                               "frac_hbm_peak": bw / (ms_w * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": bw,
                               "copy_same_bytes_us": cw}}


def run_mfma_sweep(torch):
    """The matrix-instruction probes (qa_probe.h) at 1, 2, 4 and 8 waves per
    SIMD (256 workgroups of 4 waves per step): rate of every kind."""
    from quantized_attention_quantize_amd import probes
    st = torch.cuda.current_stream()
    raw = st.cuda_stream
    sink = torch.empty(8192 * 256, dtype=torch.float32, device="cuda")
    res = {}
    for kind, (name, _) in probes.MFMA_KINDS.items():
        row = {}
        for wps in (1, 2, 4, 8):
            ops = [0.0]

            def one(i):
                ops[0] = probes.mfma(kind, 2000, 256 * wps, sink, raw)
            ms = _timed_ms(torch, one, 5, warm=1)
            row[f"{wps}_waves_per_simd"] = round(ops[0] / (ms * 1e-3) / 1e12, 1)
        res[name] = row
    return res


VARLEN_MIX = [8192, 4096, 2048, 1024, 512, 256, 128, 64, 32, 16, 8, 4, 2, 1, 1, 1]


def run_varlen(torch, qa, reps):
    """Packed sequences of 8192 down to 1 token (the pages' mixed-length
    varlen case), 32 heads, d 128, fp16, causal, in one call; beside it the
    same sequences as one dense call each (the per-sequence loop)."""
    from workloads import VarlenSpec, varlen_inputs
    spec = VarlenSpec("varlen_mix", 9, VARLEN_MIX, VARLEN_MIX, 32, 32, 128, dtype="f16")
    inp = varlen_inputs(spec)
    q, k, v = (dev_bits(torch, x, "f16") for x in (inp.q, inp.k, inp.v))
    cu_q, cu_k = torch.from_numpy(inp.cu_q).cuda(), torch.from_numpy(inp.cu_k).cuda()
    mx = max(VARLEN_MIX)
    p = qa.varlen_params(q, k, mx, mx, len(VARLEN_MIX), True)
    ws = torch.empty(qa.lib.qa_dense_sage_varlen_workspace_size(ctypes.byref(p)), dtype=torch.uint8, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    f = lambda: qa.dense_sage_attention_varlen(q, k, v, cu_q, cu_k, mx, mx, is_causal=True, workspace=ws, out=out)
    slices = [(int(a), int(b)) for a, b in zip(inp.cu_q[:-1], inp.cu_q[1:])]
    views = [(q[a:b].unsqueeze(0), k[a:b].unsqueeze(0), v[a:b].unsqueeze(0), out[a:b].unsqueeze(0))
             for a, b in slices]
    wss = [qa.dense_sage_workspace(qa.dense_params(qq, kk, True, True)) for qq, kk, _, _ in views]
    loop = lambda: [qa.dense_sage_attention(qq, kk, vv, is_causal=True, workspace=w, out=oo)
                    for (qq, kk, vv, oo), w in zip(views, wss)]

    def timed(fn):
        for _ in range(3):
            fn()
        evs = _mk_stream_events(torch, reps)
        for a, b in evs:
            a.record(); fn(); b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))
    ms, loop_ms = timed(f), timed(loop)
    qk, pv = flash_ops(VARLEN_MIX, VARLEN_MIX, 32, 128, True)
    tops = (qk + pv) / (ms * 1e-3) / 1e12
    return {"workload": f"dense_sage varlen, {len(VARLEN_MIX)} packed sequences of 8192 down to 1 token "
                        f"({sum(VARLEN_MIX)} rows), H32 d128 causal, one call (full chain)",
            "ms": ms, "TOPS": tops, "frac_int8_peak": tops / INT8_PEAK_TOPS,
            "per_sequence_loop_ms": loop_ms, "speedup_vs_loop": loop_ms / ms}


def run_practical_peaks(torch, step_bytes: int, pools: int) -> dict:
    """Practical ceilings measured on this GPU with the probes of qa_probe.h:
    a plain streaming read (1 GiB, and the decode step's byte count rotated
    over `pools` buffers as the decode bench does) and matrix-instruction
    loops of the 32x32 and 16x16 INT8/fp16 forms, and the vector-ALU rates of
    the exponential and of the fused multiply-add (best grid, median of the
    launches)."""
    from quantized_attention_quantize_amd import probes
    st = torch.cuda.current_stream()
    raw = st.cuda_stream

    def timed(fn, reps):
        fn()
        evs = _mk_stream_events(torch, reps)
        for a, b in evs:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    out = {}
    sink = torch.empty(8192 * 256, dtype=torch.float32, device="cuda")
    big = torch.ones(1 << 28, dtype=torch.int32, device="cuda")          # 1 GiB
    best = 0.0
    for wgs in (1024, 2048, 4096):
        ms = timed(lambda: probes.stream_read(big, wgs, sink, raw), 10)
        best = max(best, big.numel() * 4 / (ms * 1e-3) / 1e9)
    out["stream_read_1GiB_GBps"] = round(best, 1)
    del big
    n = step_bytes // 16 * 16
    bufs = [torch.ones(n // 4, dtype=torch.int32, device="cuda") for _ in range(pools)]
    best = 0.0
    for wgs in (256, 512, 1024):
        i = [0]

        def one():
            probes.stream_read(bufs[i[0] % pools], wgs, sink, raw)
            i[0] += 1
        ms = timed(one, 30)
        best = max(best, n / (ms * 1e-3) / 1e9)
    out["stream_read_step_bytes_GBps"] = round(best, 1)
    out["stream_read_step_bytes"] = n
    del bufs
    for kind, (name, _) in probes.MFMA_KINDS.items():
        best = 0.0
        for wgs in (512, 1024):
            ops = [0.0]

            def one():
                ops[0] = probes.mfma(kind, 4000, wgs, sink, raw)
            ms = timed(one, 5)
            best = max(best, ops[0] / (ms * 1e-3) / 1e12)
        out[f"mfma_{name}_T"] = round(best, 1)
    for kind, name in probes.VALU_KINDS.items():
        best = 0.0
        for wgs in (4096, 8192):
            ops = [0.0]

            def one():
                ops[0] = probes.valu(kind, 2048, wgs, sink, raw)
            ms = timed(one, 5)
            best = max(best, ops[0] / (ms * 1e-3) / 1e12)
        out[f"valu_{name}_T_lane_ops"] = round(best, 2)
    out["note"] = ("T = TOPS (int8) or TFLOP/s (fp16, fp8), include/qa_probe.h; valu_* in tera lane "
                   "operations per second (one exponential per score)")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--context", type=int, default=32768)
    ap.add_argument("--splits", type=int, default=0, help="split-K segments (0 = library choice)")
    ap.add_argument("--pools", type=int, default=6, help="KV pools rotated across steps")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the prefill/dense lines")
    ap.add_argument("--only", choices=["decode-batched", "decode-tiny", "producers", "prefill", "prefill-fp8", "prefill-ws", "dense",
                                       "dense-causal", "dense-fp8", "mfma-sweep"],
                    help="run one workload alone and print its line (profiling runs)")
    ap.add_argument("--reps", type=int, default=20, help="launches timed by --only")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run one plain device copy of BYTES (the reference for the memory counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_attention_quantize_amd as qa
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = args.copy_calibration // 16 * 16
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return

    if args.only:
        fns = {"decode-batched": lambda: run_decode_batched(torch, qa, args.reps, splits=args.splits or None),
               "decode-tiny": lambda: run_decode_tiny(torch, qa, args.reps),
               "producers": lambda: run_producers(torch, qa, args.reps),
               "prefill": lambda: run_prefill(torch, qa, args.reps),
               "prefill-fp8": lambda: run_prefill(torch, qa, args.reps, pv_fp8=True),
               "prefill-ws": lambda: run_prefill(torch, qa, args.reps, v_ws=True),
               "dense": lambda: run_dense(torch, qa, args.reps, False),
               "dense-causal": lambda: run_dense(torch, qa, args.reps, True),
               "dense-fp8": lambda: run_dense(torch, qa, args.reps, False, pv_fp8=True),
               "mfma-sweep": lambda: run_mfma_sweep(torch)}
        r = fns[args.only]()
        if isinstance(r, dict):
            r.pop("_ops", None)
        print(json.dumps({"only": args.only, **r}), flush=True)
        return

    spec, r = run_decode(args, torch, qa, args.warmup)
    achieved = r["step_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
    traffic = decode_traffic()
    res = {
        "metric": "INT8-QK paged attention: decode KV GB/s; prefill/dense INT8 TOPS (% peak)",
        "value": round(r["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 QK (int32 acc) / bf16 PV (fp32 acc)",   # decode: bf16 V, P as two bf16 terms
        "data": "synthetic",
        "config": {"workload": "qwen27b_decode", "num_seqs": 1, "q_heads": 24, "kv_heads": 4, "head_dim": 256,
                   "context": args.context, "block_size": 16, "k_cache": "int8 + fp32 per-token scale",
                   "v_cache": "bf16", "num_splits": r["splits"], "kv_pools_rotated": args.pools,
                   "step": "paged_decode_step: quantize the query, write the new token, split-K attention "
                           "(one kernel), then the combine kernel"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_decode (the split kernel of qa_paged_decode_step, new-token write included)",
                     "kernel_ms": round(r["kernel_ms"], 5),
                     "kernel_ms_p10_p90": [round(x, 5) for x in r["kernel_ms_p10_p90"]],
                     "algorithmic_bytes_per_launch": r["step_bytes"]},
    }
    if not args.no_extras:
        pk = run_practical_peaks(torch, r["step_bytes"], args.pools)
        res["practical_peak"] = pk
        res["roofline"]["frac_of_practical_stream"] = round(achieved / pk["stream_read_1GiB_GBps"], 4)
        rms = r["rope_ms_per_step"]
        extra = {"decode_step_rope": {
            "workload": "qwen27b decode step with rotary embedding in the split kernel (64 of 256 "
                        "channels rotated): rotate + quantize the query, rotate + write the new token, "
                        "split-K attention, combine",
            "ms": rms, "GBps": r["step_bytes"] / (rms * 1e-3) / 1e9,
            "frac_hbm_peak": r["step_bytes"] / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        runs = [("decode_2_tokens", lambda: run_decode_mt(torch, qa, args.context, 2, args.pools)),
                ("chunked_prefill", lambda: run_prefill(torch, qa, 20)),
                ("chunked_prefill_fp8pv", lambda: run_prefill(torch, qa, 20, pv_fp8=True)),
                ("chunked_prefill_v_workspace", lambda: run_prefill(torch, qa, 20, v_ws=True)),
                ("dense_sage_noncausal", lambda: run_dense(torch, qa, 10, False)),
                ("dense_sage_causal", lambda: run_dense(torch, qa, 10, True)),
                ("dense_sage_hnd_smooth_v_lse", lambda: run_dense(torch, qa, 10, False, options=True)),
                ("dense_sage_noncausal_fp8pv", lambda: run_dense(torch, qa, 10, False, pv_fp8=True)),
                ("dense_sage_causal_fp8pv", lambda: run_dense(torch, qa, 10, True, pv_fp8=True)),
                ("dense_sage_varlen_mix", lambda: run_varlen(torch, qa, 10)),
                ("decode_batched_splitk", lambda: run_decode_batched(torch, qa, 20)),
                ("decode_batched_library_splits", lambda: run_decode_batched(torch, qa, 20, splits=0)),
                ("decode_tiny", lambda: run_decode_tiny(torch, qa, 100)),
                (None, lambda: run_producers(torch, qa, 30))]
        for name, fn in runs:
            t_run = time.time()
            out = fn()
            if name is None:
                extra.update(out)
            else:
                extra[name] = out
            # one progress line per workload (stderr; stdout keeps the one JSON line)
            print(f"bench: {name or ', '.join(out)} done in {time.time() - t_run:.1f} s", file=sys.stderr, flush=True)
        res["extra"] = extra
        for e in res["extra"].values():
            if "_ops" not in e:
                continue
            # fraction of the mixed roofline at the best measured rate of each
            # operand type over the probe forms (the 16x16 forms with 16
            # independent accumulators are the fastest measured)
            qk, pv, pv_type = e.pop("_ops")
            t = e["ms"] * 1e-3
            best = lambda pre: max(v for k_, v in pk.items() if k_.startswith(pre))
            e["frac_practical_mixed"] = round((qk / (best("mfma_i8_") * 1e12) +
                                               pv / (best(f"mfma_{pv_type}_") * 1e12)) / t, 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, r["inp"], args.cpu_budget, r["out"])
    pr = torch.cuda.get_device_properties(0)
    res["device"] = {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "compute_units": pr.multi_processor_count}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
