#!/usr/bin/env python3
"""Benchmark of the block-sparse attention hot path on one MI355X.

Metric: sparse decode attention tokens/s and HBM GB/s at a 64K context
(Llama-3-8B-shaped layer, bf16, batch 8), plus block-sparse prefill TFLOP/s
at a 128K context.  One printed JSON line.

Decode.  A step is one decode step of one attention layer for the whole batch:
append the step's token K/V (retrieval heads into the paged pool, which holds
only them, with their logical page's statistics; streaming heads into a
constant-size cache of sink pages and a ring of recent pages), select pages
(every R = 4 steps, reused otherwise; the current logical page is scored from
its keys), then sparse decode attention, in two launches (lsa_decode_step: the
selection takes the new key from the step's rows, the attention kernel attends
the new token from them and writes it to its page).  --unfused times the same
step as three calls (append, select, attend).  --no-append times the step without
the append (every head in the paged pool with the window tokens already in it;
attention refreshes the statistics of the current logical page).  Steps cycle over
`--replicas` independent copies of the layer's KV pool (distinct layers of a
model), so every step reads its pages from HBM rather than from the 256 MB
last-level cache.  A cycle of replicas x R steps is captured once as a HIP
graph and replayed; the timed region covers whole cycles.

Prefill.  One call of the block-sparse prefill over 131072 tokens, 32 query
heads, 8 KV heads (4 streaming with 1 sink + 16 local tiles); the same
kernel with every head causal (the dense-causal reference of the speed-up);
and the same patterns given as static block masks (CSR lists of key tiles).

Variants (the default run is the Llama-3-8B-shaped layer with R = 4 and the
group's page scores summed): --workload llama2-7b-mha runs the multi-head
layer (32 KV heads, group size 1) in both legs, --reuse R sets the selection
interval, --aggregation max combines the group's per-head page scores by max,
--page-size / --logical-page change the page geometry of the decode pool.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, flop/s

# workload name -> (decode config, prefill config, model shape)
# name: (decode config, prefill config, layer, KV replicas by default)
WORKLOADS = {
    "llama3-8b": (2, 3, "Llama-3-8B-shaped attention layer", 8),
    "llama2-7b-mha": (6, 7, "Llama-2-7B-shaped (multi-head) attention layer", 8),
    # config 4: 64 sequences of 128K-256K tokens (about 51 GB of bf16 KV per replica)
    "llama3-8b-b64-long": (4, 3, "Llama-3-8B-shaped attention layer at batch 64, 128K-256K context", 2),
    # config 5: a 4-bit KV pool at 256K context
    "llama3-8b-kv4": (5, 3, "Llama-3-8B-shaped attention layer with a 4-bit KV pool", 8),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="llama3-8b")
    ap.add_argument("--reuse", type=int, default=None, help="selection reuse interval R (default: 4)")
    ap.add_argument("--aggregation", choices=["sum", "max"], default="sum",
                    help="how a KV head's query group combines its page scores")
    ap.add_argument("--no-append", action="store_true",
                    help="time the step without the append: every head in the paged pool (its window tokens "
                         "already written), selection + attention with the statistics refresh")
    ap.add_argument("--unfused", action="store_true",
                    help="time the appending step as three calls (append, select, attend) instead of "
                         "lsa_decode_step's two launches")
    ap.add_argument("--page-size", type=int, default=None, help="physical page size N_P of the decode pool")
    ap.add_argument("--logical-page", type=int, default=None, help="logical page size N_L of the statistics")
    ap.add_argument("--steps", type=int, default=640, help="timed decode steps (rounded up to whole cycles)")
    ap.add_argument("--warmup", type=int, default=64, help="untimed decode steps")
    ap.add_argument("--replicas", type=int, default=None,
                    help="KV pool replicas (layers) cycled through (default: 8; 2 for the batch-64 workload)")
    ap.add_argument("--prefill-reps", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill leg (profiling runs)")
    ap.add_argument("--no-causal", action="store_true",
                    help="skip the all-causal prefill reference run (profiling runs of the sparse kernel)")
    ap.add_argument("--no-csr", action="store_true",
                    help="skip the prefill run with the same patterns given as static block masks (CSR)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU sample")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--counters", action="store_true",
                    help="counter-collection run: one 1 GiB device copy (the calibration kernel), then one eager "
                         "decode cycle over the replicas; prints nothing else")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="time a plain 16384x16384x8192 bf16 torch.matmul (the vendor GEMM library) as the "
                         "practical matrix-core reference for the prefill figure, and print one JSON line")
    ap.add_argument("--hbm-reference", action="store_true",
                    help="time a plain 4 GiB device copy and a 4 GiB reduction (torch) as the reachable HBM "
                         "bandwidth reference for the decode figure, and print one JSON line")
    return ap.parse_args()


def hbm_reference(torch):
    """Large plain streams through torch: the HBM bandwidth a read+write copy
    and a read-only reduction sustain on this part."""
    n = 1 << 30                                   # 4 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    out = {}
    for name, fn, nbytes in (("copy", lambda: b.copy_(a), 2 * 4 * n), ("sum", lambda: a.sum(), 4 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "gbps": round(nbytes / ms / 1e6, 1), "frac_of_8000": round(nbytes / ms / 1e6 / 8000, 4)}
    del a, b
    out["hip_read"] = hip_read_reference(torch)
    return {"hbm": "4 GiB fp32 streams through torch; plain HIP streaming reads of 85 MB to 1 GiB", **out}


def hip_read_reference(torch):
    """A plain streaming-read kernel (block_sparse_attention_logical_amd/calib)
    over buffers of the decode launch's size and larger: what a read of that
    size sustains, ramp-up and tail included.  Eight buffers (two of 1 GiB)
    are read in turn inside a HIP graph, so no read hits the last-level cache."""
    import ctypes
    path = os.path.join(ROOT, "block_sparse_attention_logical_amd", "libcalib.so")
    lib = ctypes.CDLL(path)
    lib.calib_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    out = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    res = []
    for mb in (85, 170, 1024):
        nbuf = 2 if mb > 256 else 8
        bufs = [torch.ones(mb * 1000 * 1000 // 16 * 16, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
        for grid in (1024, 4096):
            def run():
                for b_ in bufs:
                    st = lib.calib_read_stream(b_.data_ptr(), b_.numel(), grid, out.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream)
                    if st != 0:
                        raise RuntimeError(f"calib_read_stream: hip error {st}")
            s_ = torch.cuda.Stream()
            s_.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s_):
                run()
            torch.cuda.current_stream().wait_stream(s_)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / (reps * nbuf)
            res.append({"MB": round(bufs[0].numel() / 1e6, 1), "workgroups": grid, "us": round(t * 1e6, 2),
                        "gbps": round(bufs[0].numel() / t / 1e9, 1),
                        "frac_of_8000": round(bufs[0].numel() / t / 8e12, 4)})
            del g
        del bufs
        torch.cuda.empty_cache()
    return res


def gemm_reference(torch):
    """A large bf16 GEMM through torch (hipBLASLt): what the matrix cores
    sustain on this part in a plain contraction, to set the prefill kernel's
    MFMA fraction against something reachable."""
    m, n, k = 16384, 16384, 8192
    a = torch.randn(m, k, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(k, n, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del c
    return {"gemm": f"bf16 {m}x{n}x{k} torch.matmul", "ms": round(ms, 4),
            "tflops": round(2 * m * n * k / ms / 1e9, 1), "frac_of_2500": round(2 * m * n * k / ms / 1e9 / 2500, 4)}


def counters_run(args, torch, lsa, W):
    """Kernels for rocprofv3 --pmc: a plain 1 GiB copy of known size, then the
    decode steps of one cycle (each layer read once)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    args.eager = True
    args.steps = 1
    args.warmup = 0
    bench_decode(args, torch, lsa, W)


def sha_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counters_for(kernel_tag, source_file, launch_bytes):
    """HBM traffic of one launch from the committed rocprofv3 counter summary,
    or None if it was taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != sha_of(source_file):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# decode (config 2)
# ---------------------------------------------------------------------------

def bench_decode(args, torch, lsa, W, append=True, fused=True, keep_workload=True):
    dev = "cuda"
    cfg = WORKLOADS[args.workload][0]
    R = args.reuse or W.DECODE_CONFIGS[cfg]["reuse_interval"]
    w = W.make_decode(cfg, dev, window=max(R, W.DECODE_CONFIGS[cfg]["window"]), page_size=args.page_size,
                      logical_page=args.logical_page)
    w.reuse_interval = R
    B, Hq, Hkv, D, NP = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    K = w.token_budget // NP
    agg = lsa.AGG_MAX if args.aggregation == "max" else lsa.AGG_SUM
    hd = lsa.Heads(w.head_kind, Hq, w.sink_tokens, w.local_tokens, w.sink_blocks, w.local_blocks, agg)
    nrep = max(1, args.replicas)
    lens0 = torch.tensor(w.ctx, dtype=torch.int32, device=dev)
    full = lsa.KVPool(w.dtype, w.k, w.v, Hkv, D, NP, w.logical_page, w.num_pages, k_sz=w.k_sz, v_sz=w.v_sz)
    layers = []
    for r in range(nrep):
        if append:
            # the retrieval heads in a pool of their own, the streaming heads in
            # a constant-size cache filled from the prompt (tokens < ctx)
            k, v, k_sz, v_sz = W.retrieval_pool(w)
            sink, ring = lsa.stream_cache_pages(full, hd)
            cache = lsa.StreamCache(sink, ring, *W.empty_stream_cache(w, sink, ring, fill_byte=0))
            lsa.stream_cache_fill(full, w.page_table, lens0, hd, cache)
            kv = lsa.KVPool(w.dtype, k, v, Hkv, D, NP, w.logical_page, w.num_pages, k_sz=k_sz, v_sz=v_sz,
                            stream_cache=cache)
        else:
            k = w.k if r == 0 else w.k.clone()
            v = w.v if r == 0 else w.v.clone()
            k_sz = w.k_sz if (r == 0 or w.k_sz is None) else w.k_sz.clone()
            v_sz = w.v_sz if (r == 0 or w.v_sz is None) else w.v_sz.clone()
            kv = lsa.KVPool(w.dtype, k, v, Hkv, D, NP, w.logical_page, w.num_pages, k_sz=k_sz, v_sz=v_sz)
        stats = torch.zeros(lsa.page_stats_bytes(kv, hd), dtype=torch.uint8, device=dev)
        lsa.build_page_stats(kv, w.page_table, lens0, stats, heads=hd)
        sel = torch.full((B, Hkv, K), -1, dtype=torch.int32, device=dev)
        layers.append((kv, stats, sel))
    torch.cuda.synchronize()
    lens = [w.seq_lens(s) for s in range(R)]
    rows = [W.token_rows(w, s) for s in range(R)] if append else None
    ws_sel = torch.zeros(lsa.select_pages_workspace(layers[0][0], w.page_table, lens[0], hd), dtype=torch.uint8,
                         device=dev)
    ws_dec = torch.zeros(lsa.decode_workspace(layers[0][0], w.page_table, lens[0], hd, w.token_budget),
                         dtype=torch.uint8, device=dev)
    ws_step = torch.zeros(lsa.decode_step_workspace(layers[0][0], w.page_table, lens[0], hd, w.token_budget),
                          dtype=torch.uint8, device=dev)
    out = torch.empty_like(w.q[0])
    cycle = nrep * R
    fused = fused and append

    def step(k):
        l, s = k % nrep, (k // nrep) % R
        kv, stats, sel = layers[l]
        if fused:              # append + select + attend in two launches
            lsa.decode_step(w.q[s], kv, w.page_table, lens[s], hd, rows[s][0], rows[s][1], stats, w.token_budget,
                            s, R, sel, out, ws_step, *rows[s][2:])
            return
        if append:             # the step's token, with its logical page's statistics
            lsa.append_kv(kv, w.page_table, lens[s], hd, *rows[s], stats=stats)
        lsa.select_pages(w.q[s], kv, stats, w.page_table, lens[s], hd, w.token_budget, s, R, sel, ws_sel)
        lsa.sparse_decode_attn(w.q[s], kv, w.page_table, lens[s], hd, sel, w.token_budget, out, ws_dec,
                               stats=None if append else stats)

    # warm-up (eager): every layer selects at least once
    for k in range(max(args.warmup, cycle)):
        step(k)
    torch.cuda.synchronize()

    n_cycles = max(1, math.ceil(args.steps / cycle))
    steps = n_cycles * cycle
    timing = "eager"
    graph = None
    if not args.eager:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for k in range(cycle):            # one more eager cycle on the capture stream
                    step(k)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for k in range(cycle):
                    step(k)
            graph.replay()
            torch.cuda.synchronize()
            timing = "hip-graph replay"
        except Exception as e:  # capture not available: time eager launches
            print(f"# graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graph = None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    if graph is not None:
        for _ in range(n_cycles):
            graph.replay()
    else:
        for k in range(steps):
            step(k)
    t1.record()
    torch.cuda.synchronize()
    elapsed = t0.elapsed_time(t1) / 1e3

    # per-launch duration of the decode attention kernel: the attention calls
    # of one cycle (every replica and step; with the statistics refresh, or
    # in the fused step with the append) are captured alone in a graph and
    # replayed between two HIP events on the stream they run on; without a
    # graph, events bracket eager launches held back by a spin kernel.  The
    # fused step's attention launch alone is lsa_decode_step on a step that
    # reuses the selection (decode_step 1 with reuse interval 2); writing the
    # same token again is idempotent.
    def attend(k):
        l, s = k % nrep, (k // nrep) % R
        kv, stats, sel = layers[l]
        if fused:
            lsa.decode_step(w.q[s], kv, w.page_table, lens[s], hd, rows[s][0], rows[s][1], stats, w.token_budget,
                            1, 2, sel, out, ws_step, *rows[s][2:])
            return
        lsa.sparse_decode_attn(w.q[s], kv, w.page_table, lens[s], hd, sel, w.token_budget, out, ws_dec,
                               stats=None if append else stats)

    kernel_reps = 10
    kt = None
    if graph is not None:
        try:
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2):
                for k in range(cycle):
                    attend(k)
            g2.replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(kernel_reps):
                g2.replay()
            b.record()
            torch.cuda.synchronize()
            kt = [a.elapsed_time(b) / 1e3 / (kernel_reps * cycle)]
            del g2
        except Exception as e:  # pragma: no cover
            print(f"# attention-only graph failed ({e}); timing eager launches", file=sys.stderr)
    if kt is None:
        n_kt = cycle * 4
        timers = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_kt)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.25))        # ~0.25 s at 2.4 GHz
        for k in range(n_kt):
            timers[k][0].record()
            attend(k)
            timers[k][1].record()
        torch.cuda.synchronize()
        kt = sorted(a_.elapsed_time(b_) / 1e3 for a_, b_ in timers)
    kernel_avg = sum(kt) / len(kt)

    # duration of one selection call (score kernel, fused or separate top-K):
    # the selections of one cycle (one per replica) captured alone and replayed
    sel_time = None
    if graph is not None:
        try:
            g3 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g3):
                for l in range(nrep):
                    kv, stats, sel = layers[l]
                    lsa.select_pages(w.q[0], kv, stats, w.page_table, lens[0], hd, w.token_budget, 0, R, sel,
                                     ws_sel)
            g3.replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(kernel_reps):
                g3.replay()
            b.record()
            torch.cuda.synchronize()
            sel_time = a.elapsed_time(b) / 1e3 / (kernel_reps * nrep)
            del g3
        except Exception as e:  # pragma: no cover
            print(f"# selection-only graph failed ({e})", file=sys.stderr)

    # algorithmic bytes of one attention launch: the attended keys and values
    # of every (sequence, KV head) at the measured window steps, plus q and o
    # (bytes per K or V element: 2 for bf16, 4 for f32, half a byte for int4
    # codes, whose pages also carry one fp16 (scale, zero) pair each for K and V)
    eb = {W.F32: 4, W.BF16: 2, W.INT4: 0.5}[w.dtype]
    sel_h = [layers[0][2].cpu()]
    att_tokens = att_pages = 0
    for s in range(R):
        for b in range(B):
            t = w.ctx[b] + s
            for kvh in range(Hkv):
                if w.head_kind[kvh] == 0:
                    pages = set(int(m) for m in sel_h[0][b, kvh].tolist() if m >= 0)
                    pages.add(t // NP)
                    att_tokens += sum(min(NP, t + 1 - m * NP) for m in pages)
                    att_pages += len(pages)
                else:
                    lo = max(0, t + 1 - w.local_tokens)
                    att_tokens += min(t + 1, w.sink_tokens + w.local_tokens)
                    att_pages += len({p // NP for p in range(min(w.sink_tokens, t + 1))} |
                                     set(range(lo // NP, t // NP + 1)))
    att_tokens /= R
    att_pages /= R
    kv_bytes = att_tokens * D * eb * 2 + (att_pages * 2 * 4 if w.dtype == W.INT4 else 0)
    qo_bytes = 2 * B * Hq * D * 2
    launch_bytes = kv_bytes + qo_bytes
    # whole step: + statistics refresh + selection amortised over R (the
    # statistics of every logical page of each retrieval head; int4 codes are
    # one byte per channel plus the page's (scale, zero))
    n_ret = sum(1 for x in w.head_kind if x == 0)
    lp_bytes = D + 4 / (NP // w.logical_page) if w.dtype == W.INT4 else 2 * D * eb
    sel_call_bytes = n_ret * sum(-(-(c + 1) // w.logical_page) for c in w.ctx) * lp_bytes
    sel_bytes = sel_call_bytes / R
    # the append writes one K and one V row per (sequence, KV head) and, for
    # retrieval heads, reads and writes one logical page's statistics
    app_bytes = (B * Hkv * 2 * D * eb + B * n_ret * (2 * lp_bytes)) if append else 0
    step_bytes = launch_bytes + sel_bytes + app_bytes
    if fused:              # the attention launch does the append's writes
        launch_bytes += app_bytes
    tok_s = B * steps / elapsed
    src = os.path.join(ROOT, "block_sparse_attention_logical_amd", "csrc", "decode.hip")
    # the workloads the counter summaries cover: configs 2 and 5 in their default geometry
    tag = {"llama3-8b": "cfg2", "llama3-8b-kv4": "cfg5"}.get(args.workload)
    covered = tag is not None and R == 4 and args.page_size in (None, 64) and \
        args.logical_page in (None, 16) and fused and args.aggregation == "sum"
    traffic = counters_for(f"decode_step_{tag}", src, launch_bytes) if covered else None
    sel_src = os.path.join(ROOT, "block_sparse_attention_logical_amd", "csrc", "select.hip")
    sel_traffic = counters_for(f"score_{tag}", sel_src, sel_call_bytes) if covered else None
    return dict(
        w=w if keep_workload else None, agg=args.aggregation, steps=steps, elapsed=elapsed, tok_s=tok_s, ms_per_step=elapsed / steps * 1e3,
        step_bytes=step_bytes, launch_bytes=launch_bytes, kernel_avg=kernel_avg,
        kernel_p50=kt[len(kt) // 2], timing=timing, append=append, fused=fused,
        traffic=traffic,
        traffic_source=(f"profiles/decode_step_{tag}_counters.txt, taken on decode.hip sha {sha_of(src)}"
                        if traffic is not None else None),
        sel_time=sel_time, sel_call_bytes=sel_call_bytes, sel_traffic=sel_traffic,
        sel_traffic_source=(f"profiles/score_{tag}_counters.txt, taken on select.hip sha {sha_of(sel_src)}"
                            if sel_traffic is not None else None),
    )


# ---------------------------------------------------------------------------
# prefill (config 3)
# ---------------------------------------------------------------------------

def bench_prefill(args, torch, lsa, W, O):
    dev = "cuda"
    p = W.make_prefill(WORKLOADS[args.workload][1], dev)
    kv = lsa.KVPool(p.dtype, p.k, p.v, p.num_kv_heads, p.head_dim, p.page_size, p.logical_page, p.num_pages)
    hd = lsa.Heads(p.head_kind, p.num_q_heads, 0, 1, p.sink_blocks, p.local_blocks)
    out = torch.empty_like(p.q)
    lsa.sparse_prefill_attn(p.q, kv, p.page_table, p.seq_len, hd, out)      # warm-up
    torch.cuda.synchronize()
    times = []
    for _ in range(max(1, args.prefill_reps)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        lsa.sparse_prefill_attn(p.q, kv, p.page_table, p.seq_len, hd, out)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / 1e3)
    n = -(-p.seq_len // 64)
    G = p.num_q_heads // p.num_kv_heads
    # the kernel's own count of the (query head, tile) pairs it computed, from
    # one more (untimed) call, against the oracle's block accounting
    counter = torch.zeros(1, dtype=torch.int64, device=dev)
    lsa.sparse_prefill_attn(p.q, kv, p.page_table, p.seq_len, hd, out, tile_counter=counter)
    torch.cuda.synchronize()
    kernel_tiles = int(counter.item())
    tiles = sum(G * O.block_counts(n, p.head_kind[kvh], p.sink_blocks, p.local_blocks)[0]
                for kvh in range(p.num_kv_heads))
    dense = p.num_q_heads * n * (n + 1) // 2
    flop = tiles * 4 * 64 * 64 * p.head_dim
    t = sorted(times)[len(times) // 2]
    # the same kernel with every head causal (the dense-causal reference the
    # block-sparse speed-up 1 / (1 - r) is measured against)
    causal = lsa.Heads([0] * p.num_kv_heads, p.num_q_heads, 0, 1, p.sink_blocks, p.local_blocks)
    tc = []
    for _ in range(0 if args.no_causal else max(1, min(2, args.prefill_reps))):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        lsa.sparse_prefill_attn(p.q, kv, p.page_table, p.seq_len, causal, out)
        b.record()
        torch.cuda.synchronize()
        tc.append(a.elapsed_time(b) / 1e3)
    t_causal = min(tc) if tc else float("nan")
    causal_flop = dense * 4 * 64 * 64 * p.head_dim
    # the same patterns given as static block masks (CSR lists): the general
    # iterator against the analytic one
    t_csr = float("nan")
    if not args.no_csr:
        a_idx = torch.arange(n)[:, None]
        c_idx = torch.arange(n)[None, :]
        masks = torch.stack([(c_idx <= a_idx) & ((p.head_kind[h] == 0) | (c_idx < p.sink_blocks) |
                                                 (a_idx - c_idx < p.local_blocks)) for h in range(p.num_kv_heads)])
        row_ptr, col_idx = W.csr_from_tile_masks(masks)
        del masks
        order = lsa.block_mask_schedule(row_ptr, p.num_kv_heads, p.num_q_heads, p.seq_len).to(dev)
        row_ptr, col_idx = row_ptr.to(dev), col_idx.to(dev)
        lsa.sparse_prefill_attn_csr(p.q, kv, p.page_table, p.seq_len, p.num_q_heads, row_ptr, col_idx, out,
                                    order=order)
        torch.cuda.synchronize()
        tcs = []
        for _ in range(max(1, min(2, args.prefill_reps))):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            lsa.sparse_prefill_attn_csr(p.q, kv, p.page_table, p.seq_len, p.num_q_heads, row_ptr, col_idx, out,
                                        order=order)
            b.record()
            torch.cuda.synchronize()
            tcs.append(a.elapsed_time(b) / 1e3)
        t_csr = min(tcs)
        del row_ptr, col_idx, order
    shape = dict(T=p.seq_len, Hq=p.num_q_heads, Hkv=p.num_kv_heads, D=p.head_dim,
                 n_str=sum(1 for x in p.head_kind if x == 1), sink=p.sink_blocks, local=p.local_blocks)
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(p, torch, O, args.cpu_seconds / 2, flop)
    del out, p
    torch.cuda.empty_cache()
    return dict(seconds=t, flop=flop, tiles=tiles, kernel_tiles=kernel_tiles, cpu=cpu, dense_tiles=dense,
                tflops=flop / t / 1e12,
                causal_seconds=t_causal, causal_tflops=causal_flop / t_causal / 1e12, csr_seconds=t_csr, **shape)


# ---------------------------------------------------------------------------
# oracle CPU baseline (bounded sample)
# ---------------------------------------------------------------------------

def host_details():
    """The host the oracle runs on: cores this process may use, CPU model,
    NumPy and its BLAS with the BLAS thread count."""
    import numpy as np
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = info[0].get("num_threads")
    except Exception:  # pragma: no cover
        pass
    return dict(cores=cores, cpu_model=model, numpy=np.__version__, blas=blas, blas_threads=threads)


def prefill_cpu_baseline(p, torch, O, budget_s, total_flop):
    """The oracle's block-sparse prefill on a stratified sample of query rows
    (for each of a causal and a Lambda head, rows spread evenly over the
    sequence), timed on the host; its throughput (fp64 flop of the rows'
    visible keys per second) extrapolates the whole prefill's time by flop."""
    import numpy as np
    G = p.num_q_heads // p.num_kv_heads
    table = list(range(p.page_table.numel()))
    rows_idx = p.page_table.long()
    done_flop, t_total, n_rows = 0.0, 0.0, 0
    kinds = sorted({p.head_kind[kvh]: kvh for kvh in range(p.num_kv_heads)}.items())
    strata = 512
    host = {}
    for kind, kvh in kinds:
        pool = O.Pool("bf16", p.k[rows_idx, kvh][:, None].cpu().view(torch.int16).numpy().view(np.uint16),
                      p.v[rows_idx, kvh][:, None].cpu().view(torch.int16).numpy().view(np.uint16),
                      p.page_size, p.head_dim)
        q = O.bf16_bits_to_f64(p.q[:, kvh * G].cpu().view(torch.int16).numpy().view(np.uint16))
        host[kind] = (pool.keys(table, 0, p.seq_len), pool.values(table, 0, p.seq_len), q, kvh)
    scale = 1 / np.sqrt(p.head_dim)
    k_i = 0
    while t_total < budget_s and k_i < strata:
        # stratum k_i: a row in the k_i-th of `strata` equal spans of the
        # sequence, the spans visited in bit-reversed order so that any prefix
        # of the sample spreads over the whole sequence
        j = int(format(k_i, "09b")[::-1], 2)
        row = int((j + 0.5) * p.seq_len / strata)
        for kind, (keys, values, q, kvh) in host.items():
            a = row // 64
            vis = sum(min(64 * (c + 1), row + 1) - 64 * c for c in range(a + 1)
                      if O.tile_visible(a, c, kind, p.sink_blocks, p.local_blocks))
            t0 = time.perf_counter()
            O.prefill_attention(q, keys, values, kind, 64, p.sink_blocks, p.local_blocks, scale, rows=[row])
            t_total += time.perf_counter() - t0
            done_flop += 4.0 * vis * p.head_dim
            n_rows += 1
        k_i += 1
    rate = done_flop / t_total
    return dict(value=round(rate / 1e12, 6), unit="TFLOP/s", kind="oracle", **host_details(),
                extrapolated_seconds=round(total_flop / rate, 1),
                sample=f"extrapolated: {n_rows} query rows of a causal and a Lambda head, one in each of "
                       f"{k_i} of {strata} equal spans of the {p.seq_len}-token sequence (fp64 NumPy), "
                       f"{t_total:.1f} s; the whole prefill's flop / this rate gives the extrapolated time")


def cpu_baseline(dec, torch, O, budget_s):
    import numpy as np
    w = dec["w"]
    G = w.num_q_heads // w.num_kv_heads
    spec = O.DecodeSpec(w.num_q_heads, w.num_kv_heads, list(w.head_kind), w.logical_page, w.page_size,
                        w.token_budget, w.reuse_interval, w.sink_tokens, w.local_tokens,
                        aggregation=O.MAX if dec["agg"] == "max" else O.SUM)
    done = 0
    t_total = 0.0
    i = 0
    while t_total < budget_s and i < 64:
        b = i % w.batch
        i += 1
        L = w.ctx[b] + 1
        n = -(-L // w.page_size)
        rows = w.page_table[b, :n].long()
        keys, vals = [], []
        for kvh in range(w.num_kv_heads):
            pool = O.Pool("bf16", w.k[rows, kvh][:, None].cpu().view(torch.int16).numpy().view(np.uint16),
                          w.v[rows, kvh][:, None].cpu().view(torch.int16).numpy().view(np.uint16),
                          w.page_size, w.head_dim)
            keys.append(pool.keys(list(range(n)), 0, L))
            vals.append(pool.values(list(range(n)), 0, L))
        q = O.bf16_bits_to_f64(w.q[0, b].cpu().view(torch.int16).numpy().view(np.uint16))
        t0 = time.perf_counter()
        O.decode_step(spec, q, keys, vals, None, True)       # a selection step: stats, scores, top-K, attention
        t_total += time.perf_counter() - t0
        done += 1
    # one selection step per sequence; a window of R steps selects once, so
    # the steady-state cost per token is below this selection-step cost
    return dict(value=done / t_total, unit="tokens/s", kind="oracle", **host_details(),
                sample=f"{done} decode steps with page selection, one sequence each ({w.ctx[0] // 1024}K context, "
                       f"all {w.num_kv_heads} KV heads, fp64 NumPy), {t_total:.1f} s")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(the path shards by (sequence, KV head) with no communication, "
                                   "but no multi-GPU run is built)"}))
        sys.exit(2)
    import torch
    import oracle.lsa_oracle as O
    from block_sparse_attention_logical_amd import lsa, workloads as W
    torch.cuda.set_device(0)
    lsa.load()
    if args.replicas is None:
        args.replicas = WORKLOADS[args.workload][3]

    if args.counters:
        counters_run(args, torch, lsa, W)
        return
    if args.gemm_reference:
        print(json.dumps(gemm_reference(torch)))
        return
    if args.hbm_reference:
        print(json.dumps(hbm_reference(torch)))
        return
    if args.prefill_only:
        pre = bench_prefill(args, torch, lsa, W, O)
        print(json.dumps({"prefill_ms": round(pre["seconds"] * 1e3, 3), "tflops": round(pre["tflops"], 1),
                          "all_causal_ms": round(pre["causal_seconds"] * 1e3, 3),
                          "csr_mask_ms": round(pre["csr_seconds"] * 1e3, 3),
                          "measured_speedup": round(pre["causal_seconds"] / pre["seconds"], 4)}))
        return
    dec = bench_decode(args, torch, lsa, W, append=not args.no_append, fused=not args.unfused)
    torch.cuda.empty_cache()
    # the same step as three calls (append, select, attend), and the step
    # without the append (every head in the paged pool)
    # (only the headline run keeps its workload: config 4's pool is about 51 GB)
    three = None if (args.no_append or args.unfused) else \
        bench_decode(args, torch, lsa, W, append=True, fused=False, keep_workload=False)
    torch.cuda.empty_cache()
    plain = None if args.no_append else bench_decode(args, torch, lsa, W, append=False, keep_workload=False)
    torch.cuda.empty_cache()
    pre = None if args.no_prefill else bench_prefill(args, torch, lsa, W, O)
    cpu = None if args.no_cpu_baseline else cpu_baseline(dec, torch, O, args.cpu_seconds)

    w = dec["w"]
    achieved = dec["launch_bytes"] / dec["kernel_avg"]
    model = WORKLOADS[args.workload][2]
    n_str = sum(1 for x in w.head_kind if x == 1)
    G = w.num_q_heads // w.num_kv_heads
    line = {
        "metric": "sparse decode attn tokens/s + HBM GB/s at 64K; prefill sparse TFLOP/s at 128K",
        "value": round(dec["tok_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": dec["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded; shapes of the LServe {model.split('-shaped')[0]} decode workload)",
        "config": {
            "workload": f"decode, one {model}: B={w.batch}, context "
                        f"{w.ctx[0] if min(w.ctx) == max(w.ctx) else f'{min(w.ctx)}-{max(w.ctx)}'}, "
                        f"{'int4 KV, ' if w.dtype == W.INT4 else ''}{w.num_q_heads} q heads / "
                        f"{w.num_kv_heads} KV heads ({n_str} streaming: sink {w.sink_tokens} + local "
                        f"{w.local_tokens} tokens), D={w.head_dim}, N_L={w.logical_page}, N_P={w.page_size}, "
                        f"token budget {w.token_budget}, reuse interval {w.reuse_interval}, group page scores "
                        f"combined by {args.aggregation}; " + (
                            f"one step = append of the step's K/V (retrieval heads into the paged pool with "
                            f"their statistics, streaming heads into a constant-size cache of sink + ring "
                            f"pages) + selection (every {w.reuse_interval}th step) + attention"
                            + (" in two launches (lsa_decode_step: the attention kernel appends)"
                               if dec["fused"] else " as three calls")
                            if dec["append"] else
                            f"one step = selection (every {w.reuse_interval}th step) + attention with the "
                            f"stats refresh (every head in the paged pool, window tokens pre-written)"),
            "global_batch": w.batch, "seq_len": max(w.ctx), "parallelism": "none (1 GPU)",
            "kv_replicas": args.replicas, "timing": dec["timing"],
        },
        "decode_hbm_gbps": round(dec["step_bytes"] / (dec["ms_per_step"] / 1e3) / 1e9, 1),
        "decode_step_bytes": int(dec["step_bytes"]),
        "roofline": {
            "kernel": ("lsa_decode_step: decode_mfma_kernel with the fused append" if dec["fused"] else
                       "lsa_sparse_decode_attn: decode_mfma_kernel") +
                      " (split-KV pass with the merge in its last workgroup per head)",
            "bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM, 4),
            "traffic": dec["traffic"],
            "traffic_source": dec["traffic_source"] or
            "none: no committed counter summary covers this workload on this version of decode.hip",
            "bytes_per_launch": int(dec["launch_bytes"]),
            "launch_us": round(dec["kernel_avg"] * 1e6, 2),
        },
        "cpu_baseline": cpu,
        "lsa_version": lsa.version(),
    }
    if dec["sel_time"]:
        sel_bw = dec["sel_call_bytes"] / dec["sel_time"]
        line["selection"] = {
            "kernel": "lsa_select_pages: score_kernel (top-K in its last workgroups, or topk_kernel above "
                      "4096 pages); one call every reuse interval",
            "bound": "hbm", "achieved": round(sel_bw / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(sel_bw / PEAK_HBM, 4), "bytes_per_call": int(dec["sel_call_bytes"]),
            "call_us": round(dec["sel_time"] * 1e6, 2),
            "traffic": dec["sel_traffic"],
            "traffic_source": dec["sel_traffic_source"] or
            "none: no committed counter summary covers this workload on this version of select.hip",
        }
    if three is not None:
        line["decode_three_calls"] = {
            "value": round(three["tok_s"], 1), "unit": "tokens/s", "ms_per_step": round(three["ms_per_step"], 5),
            "launch_us": round(three["kernel_avg"] * 1e6, 2),
            "frac": round(three["launch_bytes"] / three["kernel_avg"] / PEAK_HBM, 4),
            "step": "the same step as lsa_append_kv + lsa_select_pages + lsa_sparse_decode_attn",
        }
    if plain is not None:
        line["decode_without_append"] = {
            "value": round(plain["tok_s"], 1), "unit": "tokens/s", "ms_per_step": round(plain["ms_per_step"], 5),
            "launch_us": round(plain["kernel_avg"] * 1e6, 2),
            "frac": round(plain["launch_bytes"] / plain["kernel_avg"] / PEAK_HBM, 4),
            "traffic": plain["traffic"], "traffic_source": plain["traffic_source"],
            "step": "selection (every 4th step) + attention with the statistics refresh; every head in the "
                    "paged pool, window tokens already written",
        }
    if pre is not None:
        line["prefill"] = {
            "workload": f"prefill, {pre['T']} tokens, {pre['Hq']} q heads / {pre['Hkv']} KV heads "
                        f"({pre['Hkv'] - pre['n_str']} causal retrieval, {pre['n_str']} streaming with "
                        f"{pre['sink']} sink + {pre['local']} local tiles), D={pre['D']}, 64x64 tiles, bf16",
            "ms": round(pre["seconds"] * 1e3, 3),
            "tflops": round(pre["tflops"], 1),
            "nonempty_tile_heads": pre["tiles"],
            "dense_causal_tile_heads": pre["dense_tiles"],
            "theoretical_speedup": round(pre["dense_tiles"] / pre["tiles"], 4),
            "all_causal_ms": round(pre["causal_seconds"] * 1e3, 3),
            "all_causal_tflops": round(pre["causal_tflops"], 1),
            "measured_speedup": round(pre["causal_seconds"] / pre["seconds"], 4),
            "csr_mask_ms": round(pre["csr_seconds"] * 1e3, 3),
            "kernel_tile_counter": pre["kernel_tiles"],
            "tile_counter_equals_oracle": pre["kernel_tiles"] == pre["tiles"],
            "cpu_baseline": pre["cpu"],
            "roofline": {"bound": "mfma", "achieved": round(pre["tflops"], 1), "peak": PEAK_BF16 / 1e12,
                         "unit": "TFLOP/s", "frac": round(pre["tflops"] * 1e12 / PEAK_BF16, 4), "traffic": None},
        }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
