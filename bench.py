#!/usr/bin/env python3
"""Decode-attention benchmark: one paged GQA decode step per timed step.

    python bench.py [--gpus 1] [--steps 50] [--warmup 20] [--workload llama3_8b]

A step is one pass of the whole hot path, pdattn_decode + pdattn_reduce, over
one batch of seeded synthetic input already resident in HBM (in the
balanced mode the merge runs inside pdattn_decode and pdattn_reduce enqueues
nothing; --balanced times that kernel instead of the default static split +
reduce kernel). The KV pools are laid out head-major, rows
[page][kv head][slot] (--layout nhd: [page][slot][kv head]); the same step
in the other layout is timed too and reported under other_layout. Before
every timed step (outside its events) a 512 MiB buffer is rewritten, which
evicts the L2s and the 256 MB Infinity Cache, so the KV pages are read from
HBM.

Prints ONE JSON line. value = KV algorithmic bytes (every K and V element of
every valid (token, kv head) once, plus the fp8 scales) / mean step time, in
GB/s, the step timed by one event pair around decode + reduce. Warm-up runs
the timed loops' own work (flush, event records, launches). roofline = the
same bytes / the mean duration of the decode kernel alone (an event pair
around that launch on its stream, in a second flushed loop), against
MI355X's 8 TB/s HBM peak. traffic = measured HBM bytes per launch of that
kernel from the committed rocprofv3 counter summary, or null when the
kernel's sources have changed since the counters were taken. cpu_baseline =
the CPU fp64 oracle timed on this host's cores on the same step's inputs;
oracle_check = the headline outputs against that oracle's (max- and
mean-abs). configs = the tiny, long-context, many-short and FP8 KV
workloads, each timed the same way (mean, median, p10/p90, GB/s, fraction
of peak, decode and reduce kernels alone) and checked against the oracle.
device = name, gfx arch, compute units, HIP and ROCm versions.

prefill = the ragged paged prefill (pdattn_prefill) on its three workloads
(synth.PREFILL_WORKLOADS) and the ragged batch with fp8 pools, each call
timed alone after a cache flush; roofline there = algorithmic flops / mean
call time against the dense bf16 MFMA peak. fp8_kv_scales = the FP8 KV
workload's step with separate scale arrays and with inline scales. tq4 =
the Llama-3-8B-shaped step over a TQ4 compressed cache (pdattn_tq4_decode:
q rotation, chunk kernel, merge and back-rotation), GB/s of cache bytes.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "paged_kv_split_amd", "csrc")
# the sources each mode's decode kernel is built from
KERNEL_SOURCES = {
    "balanced": ["decode_dynamic.hip", "tile_ops.h", "kernels.h"],
    "static": ["decode_stream.hip", "merge_ops.h", "tile_ops.h", "kernels.h"],
}
# the static mode's decode kernel for bf16 / fp8 pools with page_size >= 16 and
# batch <= 512 (every benchmark workload)
KERNEL_NAMES = {"balanced": "decode_dynamic_kernel", "static": "decode_stream_kernel"}
# the configurations timed beside the headline, each as its own sub-record
SUB_WORKLOADS = ("tiny", "long_ctx", "many_short", "fp8_kv")
# parity bars of the decode against the oracle (out max-abs, out mean-abs, lse max-abs)
TOL = {"bf16": (1e-2, 1e-3, 1e-3), "fp8_e4m3": (4e-2, 1e-3, 1e-3)}
METRIC = "decode-attn achieved HBM GB/s + µs/call, Llama-3-8B shape, 1×MI355X"


def source_digest(mode):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[mode]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_summary_path(mode, workload, layout):
    return os.path.join(ROOT, "profiles", f"{KERNEL_NAMES[mode]}_{workload}_{layout}_hbm_traffic.txt")


def read_traffic(mode, workload, layout):
    """Bytes per launch from the committed counter summary, if it still
    describes the current kernel sources and this workload."""
    path = traffic_summary_path(mode, workload, layout)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_digest(mode) or vals.get("workload") != workload:
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def time_other_layout(pk, w, inp, args, flush, dev, reps=30):
    """The same step with the pools in the other row order (same values, same
    bytes): mean step time and rate, for comparison."""
    import torch
    import synth
    hnd = args.layout != "hnd"
    laid = synth.to_hnd(inp) if hnd else inp
    d = {k: (laid[k].to(dev) if laid[k] is not None else None)
         for k in ("q", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
    pl = pk.plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                 page_size=w.page_size, max_pages_per_seq=inp["block_table"].shape[1],
                 num_pages=inp["k_pages"].shape[0], kv_dtype=pk.KV_BF16 if w.kv_dtype == "bf16" else pk.KV_FP8_E4M3,
                 context_lens_host=inp["context_lens"], balanced=args.balanced,
                 kv_layout=pk.LAYOUT_HND if hnd else pk.LAYOUT_NHD)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    ws = pk.workspace(pl, dev)

    def step():
        pk.decode(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
                  d["context_lens"], ws, out, lse)
        pk.reduce(pl, ws, out, lse)
    for _ in range(5):
        step()
    ts = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    kvb = synth.kv_bytes(w, inp["context_lens"])
    us = statistics.fmean(ts)
    del d, ws
    return {"kv_layout": "HND" if hnd else "NHD", "us_per_call": round(us, 2),
            "gbs": round(kvb / (us * 1e-6) / 1e9, 1)}


def time_fp8_scales(pk, flush, dev, layout, reps=20):
    """The FP8 KV workload (B32, 32 q / 8 kv heads, d128, P16, L~U[1024,8192])
    with its scales in separate arrays and with each row's scale inline
    after its codes (the same values and the same bytes): mean step time
    (decode + reduce, one event pair) and KV GB/s for both."""
    import torch
    import synth
    w = synth.WORKLOADS["fp8_kv"]
    inp = synth.make_inputs(w)
    kvb = synth.kv_bytes(w, inp["context_lens"])
    res = {"workload": w.description, "kv_bytes": kvb, "kv_layout": layout.upper()}
    for name, src in (("separate", inp), ("inline", synth.to_inline(inp))):
        laid = synth.to_hnd(src) if layout == "hnd" else src
        d = {k: (laid[k].to(dev) if laid.get(k) is not None else None)
             for k in ("q", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
        pl = pk.plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                     page_size=w.page_size, max_pages_per_seq=inp["block_table"].shape[1],
                     num_pages=inp["k_pages"].shape[0], kv_dtype=pk.kv_kind(d["k_pages"]),
                     context_lens_host=inp["context_lens"],
                     kv_layout=pk.LAYOUT_HND if layout == "hnd" else pk.LAYOUT_NHD)
        out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
        lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
        ws = pk.workspace(pl, dev)

        def step():
            pk.decode(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
                      d["context_lens"], ws, out, lse)
            pk.reduce(pl, ws, out, lse)
        for _ in range(5):
            step()
        ts = []
        for i in range(reps):
            flush.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        us = statistics.fmean(ts)
        res[name] = {"us_per_call": round(us, 2), "gbs": round(kvb / (us * 1e-6) / 1e9, 1)}
        del d, ws, laid
    return res


def time_tq4(pk, flush, dev, reps=20):
    """The Llama-3-8B-shaped decode step over a TQ4 compressed cache (B32,
    32 q / 8 kv heads, d128, P16 head-major, L~U[512,4096]): the cache is
    filled by pdattn_tq4_append from the workload's bf16 rows (timed once,
    flushed), with the library's codebook; then the decode step
    (pdattn_tq4_decode: q rotation, the chunk kernel, the merge with the
    back-rotation; one event pair, caches flushed before every call), and the
    same step at the fused attention's own boundary (pdattn_tq4_decode_rotated:
    q pre-rotated, output left rotated). GB/s counts the d + 8 cache bytes of
    every valid (token, kv head) once."""
    import torch
    import synth
    w = synth.WORKLOADS["llama3_8b"]
    inp = synth.make_tq4_inputs(w)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    ck, bk = pk.tq4_codebook(w.head_dim)
    ck, bk = ck.to(dev), bk.to(dev)
    cache = d["cache"]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush.fill_(1)
    a.record()
    pk.tq4_append(d["k_new"], d["v_new"], d["token_seq"], d["token_pos"], d["block_table"], d["rotation"], bk, bk,
                  cache, num_q_heads=w.num_q_heads)
    b.record()
    torch.cuda.synchronize()
    append_us = a.elapsed_time(b) * 1e3
    nbytes = synth.tq4_kv_bytes(w, inp["context_lens"])
    prob = pk.tq4_problem(d["q"], cache, d["block_table"])
    pl = pk.tq4_plan(prob, inp["context_lens"])
    ws = torch.empty(int(pl.workspace_bytes), dtype=torch.uint8, device=dev)
    out = torch.empty(d["q"].shape, dtype=torch.float32, device=dev)
    lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=dev)

    def step():
        pk.tq4_decode(pl, d["q"], cache, d["rotation"], ck, ck, d["block_table"], d["context_lens"], ws, out, lse)
    for _ in range(5):
        step()
    ts = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    us = statistics.fmean(ts)
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("TQ4 decode produced non-finite outputs")
    # the same step at the fused attention's own boundary
    # (pdattn_tq4_decode_rotated: q pre-rotated in fp16, the output left in
    # the rotated space; the chunk kernel and the merge, no rotation kernels)
    q_rot = (d["q"].float() @ d["rotation"].t()).to(torch.float16).contiguous()
    out_r = torch.empty_like(out)

    def step_rot():
        pk.tq4_decode_rotated(pl, q_rot, cache, ck, ck, d["block_table"], d["context_lens"], ws, out_r, lse)
    for _ in range(5):
        step_rot()
    ts_r = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        a.record()
        step_rot()
        b.record()
        torch.cuda.synchronize()
        ts_r.append(a.elapsed_time(b) * 1e3)
    us_r = statistics.fmean(ts_r)
    if not bool(torch.isfinite(out_r).all()):
        raise RuntimeError("TQ4 rotated-space decode produced non-finite outputs")
    tokens = int(inp["context_lens"].sum())
    return {"workload": "Llama-3-8B-shaped TQ4 decode B32, 32 q / 8 kv heads, d128, P16 head-major, L~U[512,4096]",
            "cache_bytes": nbytes, "bf16_equivalent_bytes": synth.kv_bytes(w, inp["context_lens"]),
            "chunk_tiles": int(pl.chunk_tiles), "max_chunks": int(pl.max_chunks),
            "us_per_call": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "rotated_space_us_per_call": round(us_r, 2),
            "rotated_space_gbs": round(nbytes / (us_r * 1e-6) / 1e9, 1),
            "append_us": round(append_us, 2), "append_tokens": tokens}


def time_append(pk, w, flush, dev, layout, reps=20):
    """pdattn_kv_append timings (secondary figures, not the step): the
    decode step's append (one new token per sequence of the workload) and a
    prefill-sized append (16 sequences x 512 new tokens, in position
    order), into a bf16 pool
    and into an fp8 pool with power-of-two scales. Caches are flushed before
    every timed call; bytes are the algorithmic append bytes (bf16 rows read
    once, pool rows and scales written once)."""
    import torch
    import synth
    res = {}
    shapes = {"decode_step": dict(batch=w.batch, new_tokens=1, context=(512, 4096)),
              "prefill_16x512": dict(batch=16, new_tokens=512, context=(0, 0))}
    for sname, sh in shapes.items():
        for kv in ("bf16", "fp8_e4m3"):
            inp = synth.make_append_inputs(num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
                                           kv_dtype=kv, invalid=False, special_rows=False, spread=0, shuffle=False,
                                           seed=4000,
                                           **sh)
            laid = synth.to_hnd(inp) if layout == pk.LAYOUT_HND else inp
            d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in laid.items()}
            pow2 = kv == "fp8_e4m3"

            def call():
                pk.kv_append(d["k_new"], d["v_new"], d["token_seq"], d["token_pos"], d["block_table"],
                             d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], pow2_scales=pow2,
                             layout=layout)
            for _ in range(3):
                call()
            ts = []
            for i in range(reps):
                flush.fill_(i & 0xFF)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                call()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            rows = int(inp["token_seq"].numel()) * w.num_kv_heads
            nbytes = synth.append_bytes(rows, w.head_dim, kv)
            us = statistics.fmean(ts)
            res[f"{sname}_{'bf16' if kv == 'bf16' else 'fp8_pow2'}"] = {
                "tokens": int(inp["token_seq"].numel()), "rows": rows, "bytes": nbytes,
                "us_per_call": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del d, inp, laid
    return res


def time_multi_query(pk, w, inp, args, flush, dev, n=4, reps=30):
    """The same step with n query rows per sequence (speculative decoding's
    next_n; row i attends causally to the positions before L - (n - 1 - i)):
    the same pools and the same KV bytes, n times the queries. Mean step
    time (decode + reduce, one event pair), KV GB/s and query rows per
    second."""
    import torch
    import synth
    if w.num_q_heads // w.num_kv_heads * n > 16:
        return None
    laid = synth.to_hnd(inp) if args.layout == "hnd" else inp
    d = {k: (laid[k].to(dev) if laid[k] is not None else None)
         for k in ("k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
    g = torch.Generator().manual_seed(4300)
    q4 = torch.randn((w.batch, n, w.num_q_heads, w.head_dim), generator=g).to(torch.bfloat16).to(dev)
    pl = pk.plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                 page_size=w.page_size, max_pages_per_seq=inp["block_table"].shape[1],
                 num_pages=inp["k_pages"].shape[0], kv_dtype=pk.KV_BF16 if w.kv_dtype == "bf16" else pk.KV_FP8_E4M3,
                 context_lens_host=inp["context_lens"], q_len=n,
                 kv_layout=pk.LAYOUT_HND if args.layout == "hnd" else pk.LAYOUT_NHD)
    out = torch.empty((w.batch, n, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, n, w.num_q_heads), dtype=torch.float32, device=dev)
    ws = pk.workspace(pl, dev)

    def step():
        pk.decode(pl, q4, d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
                  d["context_lens"], ws, out, lse)
        pk.reduce(pl, ws, out, lse)
    for _ in range(5):
        step()
    ts = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    kvb = synth.kv_bytes(w, inp["context_lens"])
    us = statistics.fmean(ts)
    return {"next_n": n, "columns_per_kv_head": w.num_q_heads // w.num_kv_heads * n, "us_per_call": round(us, 2),
            "gbs": round(kvb / (us * 1e-6) / 1e9, 1),
            "query_rows_per_s": round(w.batch * n * w.num_q_heads / (us * 1e-6), 0)}


def time_d256(pk, w, args, flush, dev, reps=30):
    """The same workload with head_dim 256 (twice the KV bytes): mean step
    time (decode + reduce, one event pair) and KV GB/s."""
    import torch
    import synth
    w2 = w.with_(head_dim=256)
    inp = synth.make_inputs(w2)
    laid = synth.to_hnd(inp) if args.layout == "hnd" else inp
    d = {k: (laid[k].to(dev) if laid[k] is not None else None)
         for k in ("q", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
    pl = pk.plan(batch=w2.batch, num_q_heads=w2.num_q_heads, num_kv_heads=w2.num_kv_heads, head_dim=256,
                 page_size=w2.page_size, max_pages_per_seq=inp["block_table"].shape[1],
                 num_pages=inp["k_pages"].shape[0], kv_dtype=pk.KV_BF16 if w2.kv_dtype == "bf16" else pk.KV_FP8_E4M3,
                 context_lens_host=inp["context_lens"],
                 kv_layout=pk.LAYOUT_HND if args.layout == "hnd" else pk.LAYOUT_NHD)
    out = torch.empty((w2.batch, w2.num_q_heads, 256), dtype=torch.float32, device=dev)
    lse = torch.empty((w2.batch, w2.num_q_heads), dtype=torch.float32, device=dev)
    ws = pk.workspace(pl, dev)

    def step():
        pk.decode(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
                  d["context_lens"], ws, out, lse)
        pk.reduce(pl, ws, out, lse)
    for _ in range(5):
        step()
    ts = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    kvb = synth.kv_bytes(w2, inp["context_lens"])
    us = statistics.fmean(ts)
    del d, ws, inp, laid
    return {"kv_bytes": kvb, "us_per_call": round(us, 2), "gbs": round(kvb / (us * 1e-6) / 1e9, 1),
            "workers": pl.num_workers}


def time_merge(pk, flush, dev, reps=20):
    """pdattn_merge timings (secondary figures): a two-piece cascade (shared
    prefix + suffix) over the Llama-3-8B decode rows (32 x 32 rows, d128)
    and an eight-piece merge over the long-context rows (4 x 64 rows, d128,
    one piece per context shard). Caches flushed before every call; bytes =
    the pieces' outputs and lse read once, the merged ones written once."""
    import torch
    res = {}
    for name, S, R, D in (("cascade_2x1024_d128", 2, 1024, 128), ("shards_8x256_d128", 8, 256, 128)):
        g = torch.Generator().manual_seed(4100 + S)
        po = torch.randn((S, R, D), generator=g).to(dev)
        pl = (torch.randn((S, R), generator=g) * 4).to(dev)
        out = torch.empty((R, D), device=dev)
        lse = torch.empty((R,), device=dev)
        for _ in range(3):
            pk.merge(po, pl, out, lse)
        ts = []
        for i in range(reps):
            flush.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            pk.merge(po, pl, out, lse)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        nbytes = (S + 1) * R * (D + 1) * 4
        us = statistics.fmean(ts)
        res[name] = {"pieces": S, "rows": R, "bytes": nbytes, "us_per_call": round(us, 2),
                     "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
    return res


MFMA_BF16_PEAK_TFLOPS = 2500.0


def time_prefill(pk, flush, dev, reps=20):
    """Ragged paged prefill, one launch per call (tile maps built once per
    batch on the host, outside the timing): the three prefill workloads with
    bf16 pools, and the ragged batch with fp8 pools (separate scale arrays,
    and each row's scale inline after its codes). Each through the split
    call (pdattn_prefill_split_tiles on this device's slot count, which cuts
    long tiles where its schedule simulation says the grid ends sooner, then
    pdattn_prefill_split), and through the unsplit call (pdattn_prefill,
    longest tiles first) beside it. Caches
    flushed before every call. TFLOP/s = algorithmic flops (4 d per (query
    row, head, visible position)) / mean call time, against the dense bf16
    MFMA peak (both products run on bf16 MFMA; fp8 codes are widened)."""
    import torch
    import synth
    res = {}
    runs = [(name, "bf16") for name in sorted(synth.PREFILL_WORKLOADS)] + [("llama3_8b_prefill", "fp8_e4m3"),
                                                                            ("llama3_8b_prefill", "fp8_inline")]
    for name, kv in runs:
        inp = synth.prefill_workload(name, kv_dtype="bf16" if kv == "bf16" else "fp8_e4m3")
        if kv == "fp8_inline":
            inp = synth.to_inline(inp)
        src = synth.to_hnd(inp)
        d = {k: (src[k].to(dev) if src.get(k) is not None else None)
             for k in ("q", "qo_indptr", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
        prob = pk._prefill_problem(d["q"], d["k_pages"], d["block_table"], pk.LAYOUT_HND, None)
        rt = pk.prefill_rows_per_tile(prob)
        tb, ti = pk.prefill_tiles(inp["qo_indptr"], rt, context_lens_host=inp["context_lens"])
        tb, ti = tb.to(dev), ti.to(dev)
        st = pk.prefill_split_tiles(prob, inp["qo_indptr"], inp["context_lens"], slots=0)
        sb, si, sk = st.tile_batch.to(dev), st.tile_index.to(dev), st.tile_kv.to(dev)
        ws = pk.prefill_split_workspace(st, dev)
        out = torch.empty(d["q"].shape, dtype=torch.float32, device=dev)
        lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=dev)

        def plain():
            pk.prefill(prob, d["q"], d["qo_indptr"], tb, ti, d["k_pages"], d["v_pages"], d["k_scale"],
                       d["v_scale"], d["block_table"], d["context_lens"], out, lse)

        def split():
            pk.prefill_split(prob, d["q"], d["qo_indptr"], sb, si, sk, st.num_slots, ws, d["k_pages"], d["v_pages"],
                             d["k_scale"], d["v_scale"], d["block_table"], d["context_lens"], out, lse)

        def timed(call):
            for _ in range(3):
                call()
            ts = []
            for i in range(reps):
                flush.fill_(i & 0xFF)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                call()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            return statistics.fmean(ts)
        us_plain = timed(plain)
        us = timed(split)
        flops = synth.prefill_flops(inp["q_lens"], inp["context_lens"], prob.num_q_heads, prob.head_dim)
        tf = flops / (us * 1e-6) / 1e12
        res[f"{name}_{kv}"] = {
            "q_rows": int(inp["q_lens"].sum()), "q_lens": inp["q_lens"].tolist(),
            "context_lens": inp["context_lens"].tolist(), "tiles": int(tb.numel()), "rows_per_tile": rt,
            "workgroups": st.num_tiles * prob.num_kv_heads, "flops": flops, "us_per_call": round(us, 2),
            "tflops": round(tf, 1), "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                                 "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)},
            "split": {"entries": st.num_tiles, "slots": st.num_slots, "workspace_bytes": st.workspace_bytes},
            "unsplit_us_per_call": round(us_plain, 2),
            "outputs_finite": bool(torch.isfinite(out).all())}
        del d, out, lse, inp, src, ws
    return res


def device_info():
    """Name, gfx architecture, compute units and the HIP / ROCm versions."""
    import torch
    props = torch.cuda.get_device_properties(0)
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(path):
            with open(path) as f:
                rocm = f.read().strip()
            break
    return {"name": torch.cuda.get_device_name(0), "gfx_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hbm_bytes": props.total_memory,
            "hip_runtime": torch.version.hip, "rocm": rocm, "torch": torch.__version__}


def time_step(pk, w, inp, layout, balanced, flush, dev, steps, warmup, no_flush=False):
    """One workload's decode step on the device: plan, warm up, then time.

    Warm-up runs exactly the timed loops' work (the cache flush, the event
    records and the launches). The timed steps: a 512 MiB flush before each
    (outside its events), then one event pair around decode + reduce. Then
    each launch alone between its own events, after the same flush: the
    decode kernel's duration (for the roofline) and the reduce's. Returns the
    figures, the outputs of the last step and the plan."""
    import torch
    import synth
    laid = synth.to_hnd(inp) if layout == pk.LAYOUT_HND else inp
    d = {k: (laid[k].to(dev) if laid[k] is not None else None)
         for k in ("q", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
    pl = pk.plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                 page_size=w.page_size, max_pages_per_seq=inp["block_table"].shape[1],
                 num_pages=inp["k_pages"].shape[0],
                 kv_dtype=pk.KV_BF16 if w.kv_dtype == "bf16" else pk.KV_FP8_E4M3,
                 context_lens_host=inp["context_lens"], balanced=balanced, kv_layout=layout)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    ws = pk.workspace(pl, dev)
    if balanced:
        pk.workspace_init(pl, ws)

    def decode():
        pk.decode(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
                  d["context_lens"], ws, out, lse)

    def reduce():
        pk.reduce(pl, ws, out, lse)

    def step_loop(n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for i in range(n):
            if not no_flush:
                flush.fill_(i & 0xFF)
            ev[i][0].record()
            decode()
            reduce()
            ev[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in ev]

    def split_loop(n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for i in range(n):
            if not no_flush:
                flush.fill_(i & 0xFF)
            ev[i][0].record()
            decode()
            ev[i][1].record()
            ev[i][2].record()
            reduce()
            ev[i][3].record()
        torch.cuda.synchronize()
        return ([e[0].elapsed_time(e[1]) * 1e3 for e in ev], [e[2].elapsed_time(e[3]) * 1e3 for e in ev])

    if warmup > 0:
        step_loop(warmup)
        split_loop(warmup)
    wall0 = time.perf_counter()
    step_us = step_loop(steps)
    wall = time.perf_counter() - wall0
    dec_us, red_us = split_loop(steps)
    kvb = synth.kv_bytes(w, inp["context_lens"])
    mean_step = statistics.fmean(step_us)
    med_step = statistics.median(step_us)
    qs = statistics.quantiles(step_us, n=10) if len(step_us) > 1 else [step_us[0]] * 9
    mean_dec = statistics.fmean(dec_us)
    res = {
        "workload": w.description, "batch": w.batch, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
        "head_dim": w.head_dim, "page_size": w.page_size, "kv_dtype": w.kv_dtype, "seed": w.seed,
        "kv_layout": "HND" if layout == pk.LAYOUT_HND else "NHD", "mode": "balanced" if balanced else "static",
        "workers": pl.num_workers, "workgroups": pl.num_workgroups, "kv_bytes": kvb, "steps": steps,
        "us_per_call_mean": round(mean_step, 2), "us_per_call_median": round(med_step, 2),
        "us_per_call_p10_p90": [round(qs[0], 2), round(qs[-1], 2)],
        "gbs": round(kvb / (mean_step * 1e-6) / 1e9, 1),
        "frac": round(kvb / (mean_step * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "frac_median": round(kvb / (med_step * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_kernel_us": round(mean_dec, 2), "decode_kernel_us_median": round(statistics.median(dec_us), 2),
        "decode_kernel_frac": round(kvb / (mean_dec * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "reduce_kernel_us": round(statistics.fmean(red_us), 2),
        "reduce_kernel_us_median": round(statistics.median(red_us), 2),
        "timed_wall_s": round(wall, 4),
        "outputs_finite": bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all()),
    }
    torch.cuda.synchronize()
    return res, out.cpu(), lse.cpu(), pl


def oracle_compare(out, lse, ref_out, ref_lse, kv_dtype):
    """Max- and mean-abs differences of the device outputs from the oracle's."""
    import torch
    diff = (out.to(torch.float64) - ref_out).abs()
    fin = torch.isfinite(ref_lse)
    ldiff = float((lse.to(torch.float64)[fin] - ref_lse[fin]).abs().max()) if bool(fin.any()) else 0.0
    mx_tol, mean_tol, lse_tol = TOL[kv_dtype]
    mx, mean = float(diff.max()), float(diff.mean())
    return {"out_max_abs": mx, "out_mean_abs": mean, "lse_max_abs": ldiff,
            "tolerance": {"out_max_abs": mx_tol, "out_mean_abs": mean_tol, "lse_max_abs": lse_tol},
            "within_tolerance": bool(mx <= mx_tol and mean <= mean_tol and ldiff <= lse_tol)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle baseline (0 skips it, and the oracle checks)")
    ap.add_argument("--no-flush", action="store_true", help="time with warm caches")
    ap.add_argument("--balanced", action="store_true",
                    help="time the on-device balanced kernel instead of the static split + reduce")
    ap.add_argument("--layout", choices=("hnd", "nhd"), default="hnd",
                    help="KV pool rows [page][kv head][slot] (hnd, the default) or [page][slot][kv head] (nhd)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configurations' sub-records")
    ap.add_argument("--no-other-layout", action="store_true", help="skip the other-layout step timing")
    ap.add_argument("--no-append", action="store_true", help="skip the KV-append timings")
    ap.add_argument("--no-merge", action="store_true", help="skip the partial-state merge timings")
    ap.add_argument("--no-multi-query", action="store_true", help="skip the multi-query decode timing")
    ap.add_argument("--no-prefill", action="store_true", help="skip the ragged paged prefill timing")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 separate / inline scale timing")
    ap.add_argument("--no-tq4", action="store_true", help="skip the TQ4 compressed-cache timing")
    ap.add_argument("--no-d256", action="store_true", help="skip the head_dim 256 timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run 3 device copies of 256 MiB (a plain copy kernel of known "
                         "size, for scaling the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(each GPU would run the same kernel on its own shard of sequences or kv heads)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import paged_kv_split_amd as pk

    w = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(w)
    dev = torch.device("cuda:0")
    layout = pk.LAYOUT_HND if args.layout == "hnd" else pk.LAYOUT_NHD
    mode = "balanced" if args.balanced else "static"
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    # host planning cost (the first plan on a device also queries its occupancy)
    def make_plan():
        return pk.plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                       head_dim=w.head_dim, page_size=w.page_size,
                       max_pages_per_seq=inp["block_table"].shape[1], num_pages=inp["k_pages"].shape[0],
                       kv_dtype=pk.KV_BF16 if w.kv_dtype == "bf16" else pk.KV_FP8_E4M3,
                       context_lens_host=inp["context_lens"], balanced=args.balanced, kv_layout=layout)
    t0 = time.perf_counter()
    make_plan()
    plan_first_us = (time.perf_counter() - t0) * 1e6
    t0 = time.perf_counter()
    for _ in range(20):
        make_plan()
    plan_us = (time.perf_counter() - t0) * 1e6 / 20

    head, out, lse, pl = time_step(pk, w, inp, layout, args.balanced, flush, dev, args.steps, args.warmup,
                                   no_flush=args.no_flush)
    kv_bytes = head["kv_bytes"]
    mean_step = head["us_per_call_mean"]
    mean_dec = head["decode_kernel_us"]

    # warm-cache figure (secondary): the same step without the flush
    warm, _, _, _ = time_step(pk, w, inp, layout, args.balanced, flush, dev, 10, 3, no_flush=True)

    # streaming-read reference over a buffer of the step's KV size
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    rbytes = (kv_bytes // 4096) * 4096
    rbuf = torch.ones(rbytes, dtype=torch.uint8, device=dev)
    sink = pk.stream_read_sink(num_cus, dev)
    rt = []
    for i in range(12):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pk.stream_read(rbuf, sink, num_cus)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            rt.append(a.elapsed_time(b) * 1e3)
    ceiling = rbytes / (statistics.median(rt) * 1e-6) / 1e9
    del rbuf
    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            flush.fill_(0)
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the other configurations, each timed like the headline
    configs = {}
    sub_out = {}
    if not args.no_configs:
        for name in SUB_WORKLOADS:
            if name == args.workload:
                continue
            sw = synth.WORKLOADS[name]
            sinp = synth.make_inputs(sw)
            res, so, sl, _ = time_step(pk, sw, sinp, layout, args.balanced, flush, dev, max(args.steps, 20),
                                       args.warmup, no_flush=args.no_flush)
            configs[name] = res
            sub_out[name] = (sw, sinp, so, sl)
            torch.cuda.empty_cache()

    other = None if args.no_other_layout else time_other_layout(pk, w, inp, args, flush, dev)
    append = None if args.no_append else time_append(pk, w, flush, dev, layout)
    merge = None if args.no_merge else time_merge(pk, flush, dev)
    multi = None if args.no_multi_query else time_multi_query(pk, w, inp, args, flush, dev)
    d256 = None if args.no_d256 else time_d256(pk, w, args, flush, dev)
    prefill = None if args.no_prefill else time_prefill(pk, flush, dev)
    fp8_scales = None if args.no_fp8 else time_fp8_scales(pk, flush, dev, args.layout)
    tq4 = None if args.no_tq4 else time_tq4(pk, flush, dev)

    # the cpu_baseline leg: the CPU fp64 oracle, timed on this host's cores on
    # the headline step's inputs; its outputs also check the device's
    cpu = None
    parity = None
    if args.cpu_seconds > 0:
        import oracle
        times = []
        threads = 0
        start = time.perf_counter()
        while True:
            t = time.perf_counter()
            ref_out, ref_lse, threads = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                                                      inp["context_lens"], k_scale=inp["k_scale"],
                                                      v_scale=inp["v_scale"], return_threads=True)
            times.append(time.perf_counter() - t)
            if time.perf_counter() - start >= args.cpu_seconds:
                break
        per_call = statistics.median(times)
        cpu = {"value": round(kv_bytes / per_call / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the full {w.name} step ({w.batch} sequences) repeated {len(times)} times "
                         f"({sum(times):.1f} s); median {per_call * 1e6:.0f} us/call"}
        parity = oracle_compare(out, lse, ref_out, ref_lse, w.kv_dtype)

        def single_thread(sw, sinp, budget):
            # the same oracle on one thread, over a bounded prefix of the batch
            nb = max(1, min(sw.batch, 4))
            t1 = []
            begin = time.perf_counter()
            while True:
                t = time.perf_counter()
                oracle.decode(sinp["q"][:nb], sinp["k_pages"], sinp["v_pages"], sinp["block_table"][:nb],
                              sinp["context_lens"][:nb], k_scale=sinp["k_scale"], v_scale=sinp["v_scale"],
                              threads=1)
                t1.append(time.perf_counter() - t)
                if time.perf_counter() - begin >= budget:
                    break
            sub_bytes = synth.kv_bytes(sw, sinp["context_lens"][:nb])
            return {"value": round(sub_bytes / statistics.median(t1) / 1e9, 4), "unit": "GB/s", "cores": 1,
                    "kind": "oracle", "sample": f"the first {nb} sequences of the step, {len(t1)} calls"}

        cpu["single_thread"] = single_thread(w, inp, min(3.0, args.cpu_seconds))
        for name, (sw, sinp, so, sl) in sub_out.items():
            ro, rl = oracle.decode(sinp["q"], sinp["k_pages"], sinp["v_pages"], sinp["block_table"],
                                   sinp["context_lens"], k_scale=sinp["k_scale"], v_scale=sinp["v_scale"])
            configs[name]["oracle_check"] = oracle_compare(so, sl, ro, rl, sw.kv_dtype)
            if name in ("tiny", "many_short"):
                configs[name]["cpu_single_thread"] = single_thread(sw, sinp, min(3.0, args.cpu_seconds))

    traffic = read_traffic(mode, w.name, args.layout)
    # fp8 pools: the two fp32 scales per (token, kv head) inside kv_bytes
    scale_bytes = (int(inp["context_lens"].to(torch.int64).sum()) * w.num_kv_heads * 8
                   if w.kv_dtype == "fp8_e4m3" else 0)
    achieved = kv_bytes / (mean_dec * 1e-6) / 1e9
    rec = {
        "metric": METRIC,
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_step / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.description, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
                   "context_lens": list(w.lens[1:]) if w.lens[0] == "uniform" else list(w.lens[1]),
                   "seed": w.seed, "kv_layout": args.layout.upper(), "workers": pl.num_workers,
                   "workgroups": pl.num_workgroups, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "oracle_check": parity,
        "us_per_call": round(mean_step, 2),
        "us_per_call_median": head["us_per_call_median"],
        "us_per_call_p10_p50_p90": [head["us_per_call_p10_p90"][0], head["us_per_call_median"],
                                    head["us_per_call_p10_p90"][1]],
        "frac_of_peak_step_mean": head["frac"],
        "frac_of_peak_step_median": head["frac_median"],
        "mode": mode,
        "decode_kernel_us": head["decode_kernel_us"],
        "decode_kernel_us_median": head["decode_kernel_us_median"],
        "reduce_kernel_us": head["reduce_kernel_us"],
        "reduce_kernel_us_median": head["reduce_kernel_us_median"],
        "warm_cache_us_per_call": warm["us_per_call_median"],
        "kv_bytes_per_call": kv_bytes,
        "kv_payload_bytes_per_call": kv_bytes - scale_bytes,
        "value_payload_only_gbs": round((kv_bytes - scale_bytes) / (mean_step * 1e-6) / 1e9, 1),
        "stream_read_ceiling_gbs": round(ceiling, 1),
        "frac_of_stream_read_ceiling": round(kv_bytes / (mean_step * 1e-6) / 1e9 / ceiling, 4),
        "plan_host_us": round(plan_us, 1),
        "plan_host_first_call_us": round(plan_first_us, 1),
        "timed_wall_s": head["timed_wall_s"],
        "cache_flush_between_steps": not args.no_flush,
        "outputs_finite": head["outputs_finite"],
        "device": device_info(),
        "kernel_source_sha256_16": source_digest(mode),
        "configs": configs,
        "other_layout": other,
        "kv_append": append,
        "merge": merge,
        "multi_query": multi,
        "head_dim_256": d256,
        "prefill": prefill,
        "fp8_kv_scales": fp8_scales,
        "tq4": tq4,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
