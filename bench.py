#!/usr/bin/env python3
"""MLA latent-cache decode benchmark on one MI355X.

One step = the whole decode hot path for one batch: mla_absorb_q ->
mla_decode (split-KV) -> mla_combine -> mla_out_proj, on the DeepSeek-V2
shaped workload (128 heads, d_c 512, rotary 64, batch 32, every sequence 4096
tokens, bf16 cache). Inputs are seeded synthetic tensors already resident in
HBM. The timed region replays HIP graphs of whole steps; the latent cache is
rotated over several copies (>= 600 MB in all) so the 256 MB Infinity Cache
cannot hold it between steps.

Prints one JSON line: queries/s of the step (value), the decode kernel's
latent-cache bandwidth against the 8 TB/s HBM peak (roofline; its duration
from the event pair each decode launch carries within eagerly launched
steps), and
the CPU oracle timed on a bounded sample on this host (cpu_baseline).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode queries/sec + latent-cache HBM GB/s (% peak) at B=32, L=4096 bf16"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv2_b32_l4096")
    ap.add_argument("--splits", type=int, default=0, help="0 = library suggestion")
    ap.add_argument("--eager", action="store_true", help="launch from Python instead of graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy-mb", type=int, default=512,
                    help="size of the plain copy run once for byte-counter calibration")
    return ap.parse_args()


def hbm_traffic(workload):
    """HBM bytes per decode launch from the committed byte-counter profile of
    this workload (rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by what it
    reads on a plain copy of known size), or None when there is none or the
    kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "mla_decode_%s_hbm_bytes.json" % workload)
    if not os.path.exists(path):
        return None
    prof = json.load(open(path))
    h = hashlib.sha256()
    for f in prof["source_files"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != prof["source_sha256"]:
        return None
    return int(round(prof["bytes_per_launch"]))


def cache_append_time(inp, stream, reps=20, per_graph=20):
    """mla_cache_append (the new token's latent and rotary key, written into
    the cache) for the workload's batch and the DeepSeek-V2 hidden size 5120,
    bf16: HIP events on its stream around replays of a graph of back-to-back
    calls. Not part of the decode step; reported beside it."""
    import torch
    import mla_latent_kv_28_amd as mla
    from mla_synth import make_append_inputs
    d, B = inp.dims, inp.batch
    a = make_append_inputs(d, batch=B, seed=1, max_position=1, positions=[0] * B)
    dev = "cuda:0"
    h, w1, w2 = a.h.to(dev), a.w_dkv.to(dev), a.w_kr.to(dev)
    pos = torch.from_numpy(a.positions).to(dev)
    rows = torch.zeros((B, d.d_latent + d.d_rope), dtype=torch.bfloat16, device=dev)
    cache = mla.kv_cache(mla.BF16, rows, seq_stride=1)
    ws = torch.empty(mla.mla_cache_append_workspace(d, B, d.hidden) // 4, dtype=torch.float32, device=dev)

    def call():
        mla.mla_cache_append(d, B, d.hidden, h, w1, w2, None, mla.BF16, a.eps, a.base, pos, cache, ws)

    with torch.cuda.stream(stream):
        for _ in range(3):
            call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(per_graph):
            call()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
    # bytes that must move: both projections, the hidden states, the rows written
    alg = (d.d_latent + d.d_rope) * d.hidden * 2 + B * d.hidden * 2 + B * (d.d_latent + d.d_rope) * 2
    gbps = alg / (us * 1e-6) / 1e9
    return {"batch": B, "hidden": d.hidden, "cache": "bf16", "us_per_call": round(us, 3),
            "calls_timed": reps * per_graph, "algorithmic_bytes": alg, "GBps": round(gbps, 1),
            "frac_of_8TBps": round(gbps / HBM_PEAK_GBPS, 4),
            "timing": "HIP events on the launch stream around graph replays of back-to-back calls"}


def o_proj_time(inp, stream, reps=10, copies=3):
    """mla_o_proj (u = W_O [o_1; ...; o_H]) for the workload's batch, bf16,
    hidden 5120: HIP events on its stream around replays of a graph of calls
    that rotate over `copies` copies of W_O (168 MB each, together beyond the
    256 MB Infinity Cache). Not part of the decode step; reported beside it."""
    import torch
    import mla_latent_kv_28_amd as mla
    from mla_synth import make_oproj_inputs
    d, B = inp.dims, inp.batch
    o, w_o = make_oproj_inputs(d, B, seed=2)
    o = o.to("cuda:0")
    ws = [w_o.to("cuda:0")] + [None] * (copies - 1)
    for i in range(1, copies):
        ws[i] = ws[0].clone()
    out = torch.empty((B, d.hidden), dtype=torch.bfloat16, device="cuda:0")
    work = torch.empty(mla.mla_o_proj_workspace(d, B, d.hidden) // 4, dtype=torch.float32, device="cuda:0")
    per_graph = 4 * copies

    def call(i):
        mla.mla_o_proj(d, B, d.hidden, o, ws[i % copies], mla.BF16, out, mla.BF16, work)

    with torch.cuda.stream(stream):
        for i in range(copies):
            call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(per_graph):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
    k = d.num_heads * d.d_v
    alg = d.hidden * k * 2 + B * k * 2 + B * d.hidden * 2
    gbps = alg / (us * 1e-6) / 1e9
    del ws
    return {"batch": B, "hidden": d.hidden, "k": k, "us_per_call": round(us, 3), "calls_timed": reps * per_graph,
            "weight_copies_rotated": copies, "algorithmic_bytes": alg, "GBps": round(gbps, 1),
            "frac_of_8TBps": round(gbps / HBM_PEAK_GBPS, 4),
            "timing": "HIP events on the launch stream around graph replays of back-to-back calls"}


def _graph_time(stream, call, reps, per_graph):
    """Microseconds per call: HIP events on `stream` around `reps` replays of
    a graph of `per_graph` back-to-back calls (call(i), i = 0 .. per_graph-1)."""
    import torch
    with torch.cuda.stream(stream):
        for i in range(2):
            call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(per_graph):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * per_graph)


def query_proj_time(inp, stream, reps=10, per_graph=20, copies=4):
    """mla_query_proj (c_Q = RMSNorm(W_DQ h), q^C = W_UQ c_Q, q^R with YaRN
    rotation) for the workload's batch, hidden 5120, d'_c 1536, bf16: HIP
    events on its stream around replays of a graph of calls that rotate over
    `copies` copies of the three weights (91 MB a copy, together beyond the
    256 MB Infinity Cache). Not part of the decode step (its output feeds the
    absorb); reported beside it."""
    import torch
    import mla_latent_kv_28_amd as mla
    from mla_synth import make_query_inputs
    d, B = inp.dims, inp.batch
    q = make_query_inputs(d, batch=B, seed=3, max_position=163840)
    dev = "cuda:0"
    h = q.h.to(dev)
    w = [tuple(t.to(dev) for t in (q.w_dq, q.w_uq, q.w_qr))]
    for _ in range(copies - 1):
        w.append(tuple(t.clone() for t in w[0]))
    pos = torch.from_numpy(q.positions).to(dev)
    qn = torch.empty((B, d.num_heads, d.d_nope), dtype=torch.bfloat16, device=dev)
    qr = torch.empty((B, d.num_heads, d.d_rope), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.mla_query_proj_workspace(d, B, d.hidden, q.d_qlatent), dtype=torch.uint8, device=dev)
    rope = mla.Rope(10000.0, 40.0, 1.0, 32.0, 4096)

    def call(i):
        w_dq, w_uq, w_qr = w[i % copies]
        mla.mla_query_proj(d, B, d.hidden, q.d_qlatent, h, w_dq, None, w_uq, w_qr, mla.BF16, q.eps, rope, pos,
                           qn, qr, ws)

    us = _graph_time(stream, call, reps, per_graph)
    n2 = d.num_heads * (d.d_nope + d.d_rope)
    alg = (q.d_qlatent * d.hidden + n2 * q.d_qlatent) * 2 + B * d.hidden * 2 + B * n2 * 2
    gbps = alg / (us * 1e-6) / 1e9
    del w
    return {"batch": B, "hidden": d.hidden, "d_qlatent": q.d_qlatent, "us_per_call": round(us, 3),
            "calls_timed": reps * per_graph, "weight_copies_rotated": copies, "algorithmic_bytes": alg,
            "GBps": round(gbps, 1), "frac_of_8TBps": round(gbps / HBM_PEAK_GBPS, 4),
            "timing": "HIP events on the launch stream around graph replays of back-to-back calls"}


def prefill_time(pipe, stream, seqs=4, reps=5, per_graph=2):
    """mla_prefill over whole 4096-token prompts of the first `seqs`
    sequences of the workload's cache, queries drawn from torch's seeded
    generator as N(0, 0.3^2) (their values do not change the work). The path
    is MFMA-bound: reported against the bf16 dense peak, with the flops of
    the up-projections and of the causal (query, key) pairs."""
    import torch
    import mla_latent_kv_28_amd as mla
    d = pipe.dims
    L = pipe.max_seq_len
    n = L
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(5)
    qn = (torch.randn((seqs * n, d.num_heads, d.d_nope), generator=gen, device=dev) * 0.3).to(torch.bfloat16)
    qr = (torch.randn((seqs * n, d.num_heads, d.d_rope), generator=gen, device=dev) * 0.3).to(torch.bfloat16)
    lens = torch.full((seqs,), L, dtype=torch.int32, device=dev)
    out = torch.empty((seqs * n, d.num_heads, d.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((seqs * n, d.num_heads), dtype=torch.float32, device=dev)
    ws = torch.empty(mla.mla_prefill_workspace(d, seqs, L), dtype=torch.uint8, device=dev)

    def call(i):
        mla.mla_prefill(d, seqs, n, qn, qr, pipe.cache, lens, L, pipe.w_uk, pipe.w_uv, pipe.sm_scale, out, lse, ws)

    us = _graph_time(stream, call, reps, per_graph)
    H = d.num_heads
    up = 2 * 2 * seqs * L * d.d_latent * H * d.d_nope                   # K^C and V^C of every row
    pairs = seqs * n * (n + 1) // 2                                      # causal (query, key) pairs
    att = pairs * H * 2 * ((d.d_nope + d.d_rope) + d.d_v)
    tflops = (up + att) / (us * 1e-6) / 1e12
    del ws, out, qn, qr
    return {"sequences": seqs, "prompt_tokens": n, "us_per_call": round(us, 1), "calls_timed": reps * per_graph,
            "gflop_per_call": round((up + att) / 1e9, 1), "tflops": round(tflops, 1),
            "frac_of_bf16_dense_peak": round(tflops / 2500.0, 4),
            "tokens_per_s": round(seqs * n / (us * 1e-6), 1),
            "timing": "HIP events on the launch stream around graph replays of back-to-back calls"}


def multi_token_time(pipe, caches, stream, n=2, reps=20):
    """mla_decode_multi with n new tokens per sequence over the workload's
    cache (the absorbed queries of the step, each repeated n times), rotating
    the cache copies: the decode launch's time, query rows per second and the
    cache bandwidth counted on the bytes of distinct cached rows."""
    import torch
    import mla_latent_kv_28_amd as mla
    d, B, S = pipe.dims, pipe.seqs, pipe.num_splits
    q = pipe.q_lat.repeat_interleave(n, dim=0).contiguous()
    out = torch.empty((B * n, S, d.num_heads, d.d_latent), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((B * n, S, d.num_heads), dtype=torch.float32, device="cuda:0")
    nb = len(caches)

    def call(i):
        mla.mla_decode_multi(d, B, n, q, caches[i % nb], pipe.seq_lens, pipe.max_seq_len, pipe.sm_scale, S, out,
                             lse, mla.BF16)

    us = _graph_time(stream, call, reps, nb)
    tokens = int(pipe.seq_lens.to(torch.int64).sum().item())
    alg = tokens * (d.d_latent + d.d_rope) * 2
    gbps = alg / (us * 1e-6) / 1e9
    return {"tokens_per_seq": n, "query_rows": B * n, "splits": S, "us_per_launch": round(us, 3),
            "query_rows_per_s": round(B * n / (us * 1e-6), 1), "cache_GBps": round(gbps, 1),
            "frac_of_8TBps": round(gbps / HBM_PEAK_GBPS, 4),
            "timing": "HIP events on the launch stream around graph replays of decode launches alone"}


def layer_time(inp, pipe, caches, stream, copies=2, reps=5):
    """One whole MLA layer for one new token per sequence, at the workload's
    batch and the DeepSeek-V2 hidden size 5120: the query path and the cache
    append of the new token (at position L - 1, the row the decode then reads),
    the decode step of the benchmark (absorb, decode, merge + W_UV) and W_O.
    The append depends only on the hidden state, like the query path, so it
    can also run on a second stream beside it (default priority; forked from
    and joined back to the launch stream); both forms are timed, the one-stream
    form is reported as the layer's time. HIP events around replays of graphs of
    layers rotating `copies` copies of every weight and the step's cache
    copies."""
    import math as _m
    import torch
    import mla_latent_kv_28_amd as mla
    from mla_synth import make_append_inputs, make_oproj_inputs, make_query_inputs
    d, B, dev = inp.dims, pipe.batch, "cuda:0"
    lens = pipe.seq_lens.to(torch.int32)
    q = make_query_inputs(d, batch=B, seed=3)
    a = make_append_inputs(d, batch=B, seed=4)
    _, w_o = make_oproj_inputs(d, B, seed=2)
    h = q.h.to(dev)
    base = dict(w_dq=q.w_dq, w_uq=q.w_uq, w_qr=q.w_qr, w_dkv=a.w_dkv, w_kr=a.w_kr, w_uk=pipe.w_uk.cpu(),
                w_uv=pipe.w_uv.cpu(), w_o=w_o)
    W = [{k: v.to(dev).contiguous() for k, v in base.items()} for _ in range(copies)]
    qn = torch.empty((B, d.num_heads, d.d_nope), dtype=torch.bfloat16, device=dev)
    qr = torch.empty((B, d.num_heads, d.d_rope), dtype=torch.bfloat16, device=dev)
    u = torch.empty((B, d.hidden), dtype=torch.bfloat16, device=dev)
    pos = (lens - 1).contiguous()
    ws_q = torch.empty(mla.mla_query_proj_workspace(d, B, d.hidden, q.d_qlatent), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(mla.mla_cache_append_workspace(d, B, d.hidden) // 4, dtype=torch.float32, device=dev)
    ws_o = torch.empty(mla.mla_o_proj_workspace(d, B, d.hidden) // 4, dtype=torch.float32, device=dev)
    rope = mla.Rope(10000.0, 40.0, 1.0, 32.0, 4096)
    saved = (pipe.q_nope, pipe.q_rope, pipe.w_uk, pipe.w_uv, pipe.cache)
    pipe.q_nope, pipe.q_rope = qn, qr
    nb = len(caches)
    per_graph = copies * nb // _m.gcd(copies, nb)
    side = torch.cuda.Stream()

    def layer(i, overlap):
        w, cache = W[i % copies], caches[i % nb]
        main = torch.cuda.current_stream()

        def append():
            mla.mla_cache_append(d, B, d.hidden, h, w["w_dkv"], w["w_kr"], None, mla.BF16, a.eps, rope, pos,
                                 cache, ws_a)
        if overlap:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                append()
        mla.mla_query_proj(d, B, d.hidden, q.d_qlatent, h, w["w_dq"], None, w["w_uq"], w["w_qr"], mla.BF16, q.eps,
                           rope, pos, qn, qr, ws_q)
        if overlap:
            main.wait_stream(side)
        else:
            append()
        pipe.w_uk, pipe.w_uv, pipe.cache = w["w_uk"], w["w_uv"], cache
        pipe.run()
        mla.mla_o_proj(d, B, d.hidden, pipe.out, w["w_o"], mla.BF16, u, mla.BF16, ws_o)

    res = {}
    try:
        for overlap in (True, False):
            with torch.cuda.stream(stream):
                for i in range(per_graph):
                    layer(i, overlap)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(per_graph):
                    layer(i, overlap)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            res[overlap] = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
            del g
    finally:
        pipe.q_nope, pipe.q_rope, pipe.w_uk, pipe.w_uv, pipe.cache = saved
    us = res[False]
    return {"batch": B, "hidden": d.hidden, "us_per_layer": round(us, 3), "queries_per_s": round(B / (us * 1e-6), 1),
            "us_per_layer_append_on_second_stream": round(res[True], 3), "layers_timed": reps * per_graph,
            "weight_copies_rotated": copies,
            "kernels": "query path, cache append, absorb, decode, merge + W_UV, W_O (one stream)",
            "timing": "HIP events on the launch stream around graph replays of back-to-back layers"}


def cpu_baseline(inp, budget_s):
    """The float64 oracle, as it stands, on whole sequences of the same
    workload until about `budget_s` seconds of CPU work have run."""
    import numpy as np
    import oracle
    from mla_synth import oracle_args
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    a = oracle_args(inp)
    done, t0 = 0, time.perf_counter()
    while done < inp.batch:
        L = int(inp.seq_lens[done])
        c_kv, k_rope = oracle.gather_rows(a["cache"], done, L)
        oracle.attend_nonabsorbed(c_kv, k_rope, a["q_nope"][done], a["q_rope"][done],
                                  a["w_uk"], a["w_uv"], a["sm_scale"])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d sequences (all %d heads, %d tokens each), %.1f s, float64 "
                      "non-absorbed oracle" % (done, inp.batch, inp.dims.num_heads,
                                               int(inp.seq_lens[0]), dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU mode "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mla_latent_kv_28_amd as mla
    from mla_latent_kv_28_amd.pipeline import DecodePipeline
    from mla_synth import make_inputs

    mla.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = make_inputs(args.workload)
    B, L = inp.batch, inp.max_seq_len
    cache_bytes = inp.cache_bytes()
    pipe = DecodePipeline(inp, num_splits=args.splits or None, device="cuda:0")
    S = pipe.num_splits

    # rotate copies of the cache so that the working set exceeds the MALL
    nbuf = max(4, math.ceil(2.3 * MALL_BYTES / max(cache_bytes, 1)))
    if inp.dtype == "fp8":
        copies = [(pipe.codes, pipe.rope, pipe.scale)] + [
            (pipe.codes.clone(), pipe.rope.clone(), pipe.scale.clone()) for _ in range(nbuf - 1)]
        caches = [mla.kv_cache(mla.FP8_E4M3, c, rope=r, scale=s, row_stride=inp.dims.d_latent,
                               rope_stride=inp.dims.d_rope, page_size=pipe.cache.page_size,
                               seq_stride=pipe.cache.seq_stride, block_table=pipe.block_table,
                               max_pages_per_seq=pipe.cache.max_pages_per_seq) for c, r, s in copies]
    else:
        copies = [pipe.rows] + [pipe.rows.clone() for _ in range(nbuf - 1)]
        caches = [mla.kv_cache(pipe.compute, r, row_stride=inp.dims.width,
                               page_size=pipe.cache.page_size, seq_stride=pipe.cache.seq_stride,
                               block_table=pipe.block_table,
                               max_pages_per_seq=pipe.cache.max_pages_per_seq) for r in copies]

    stream = torch.cuda.Stream()

    def step(i):
        pipe.cache = caches[i % nbuf]
        pipe.run()

    # graphs: one whole step per cache copy
    graphs = {}
    if not args.eager:
        with torch.cuda.stream(stream):
            for i in range(nbuf):       # warm the launch path before capture
                step(i)
        torch.cuda.synchronize()
        for name, fn in (("step", step),):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(nbuf):
                    fn(i)
            graphs[name] = g

    def run(name, fn, n):
        """n replays of `name` (each = nbuf launches of fn) or eager calls."""
        if not args.eager:
            for _ in range(n):
                graphs[name].replay()
        else:
            with torch.cuda.stream(stream):
                for i in range(n * nbuf):
                    fn(i)

    def timed(name, fn, steps, warmup):
        reps = max(1, math.ceil(steps / nbuf))
        wreps = max(1, math.ceil(warmup / nbuf))
        run(name, fn, wreps)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            run(name, fn, reps)
            e1.record(stream)
        torch.cuda.synchronize()
        n = reps * nbuf
        return e0.elapsed_time(e1) / n, n       # ms per launch set, count

    # A plain device-to-device copy of known size: hardware byte counters
    # (FETCH_SIZE / WRITE_SIZE) read on it calibrate those read on the decode.
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb << 18
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def read_probe_gbps(nbytes=1 << 30, reps=20):
        """Read bandwidth of a plain streaming read (mla_read_probe) of a
        1 GiB buffer, 20 back-to-back launches between two events."""
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        sink = torch.zeros(4, dtype=torch.float32, device=dev)
        with torch.cuda.stream(stream):
            for _ in range(3):
                mla.mla_read_probe(buf, sink, stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                mla.mla_read_probe(buf, sink, stream)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        del buf, sink
        return nbytes / (ms * 1e-3) / 1e9

    def in_step_kernel_times(n):
        """The decode kernel's execution time, and that of the rest of the step
        (split merge and out-projection, one fused call where the pipeline uses
        it), in n whole steps launched eagerly on the bench stream: each timed
        launch carries its HIP event pair (mla_time_next_launch, i.e.
        hipExtLaunchKernel). A spin kernel of about 20 ms goes first, so that
        all n steps are queued before the GPU reaches them and run back to
        back. The events' own packets add a few microseconds per interval (the
        start timestamp is taken as the previous kernel ends), so the figure
        is slightly above the kernel's execution interval as a profiler reports
        it: a conservative duration."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for row in ev:
            for e in row:
                e.record(stream)          # torch creates its events lazily
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(2 * nbuf):
                step(i)
            torch.cuda._sleep(int(4e7))
            for i in range(n):
                pipe.cache = caches[i % nbuf]
                pipe.absorb()
                mla.mla_time_next_launch(ev[i][0], ev[i][1])
                pipe.decode()
                if pipe.fused:
                    mla.mla_time_next_launch(ev[i][2], ev[i][3])
                    pipe.combine_out_proj()
                else:
                    mla.mla_time_next_launch(ev[i][2], None)
                    pipe.combine()
                    mla.mla_time_next_launch(None, ev[i][3])
                    pipe.out_proj()
        torch.cuda.synchronize()
        decs = sorted(e[0].elapsed_time(e[1]) for e in ev)
        rest = sum(e[2].elapsed_time(e[3]) for e in ev) / n
        pct = {q: decs[min(n - 1, int(round(q / 100.0 * (n - 1))))] for q in (10, 50, 90)}
        return sum(decs) / n, rest, pct

    torch.cuda.synchronize()
    probe_gbps = read_probe_gbps()
    ms_step, nsteps = timed("step", step, args.steps, args.warmup)
    ms_dec, ms_rest, dec_pct = in_step_kernel_times(max(args.steps, 100))

    q_step = B / (ms_step * 1e-3)
    gbps_step = cache_bytes / (ms_step * 1e-3) / 1e9
    gbps_dec = cache_bytes / (ms_dec * 1e-3) / 1e9
    # scores over d_c + d_rope and the latent sum over d_c, per cached token and head
    tokens = int(inp.seq_lens.astype(np.int64).sum())
    flops_dec = tokens * 2 * inp.dims.num_heads * (inp.dims.width + inp.dims.d_latent)

    result = {
        "metric": METRIC,
        "value": round(q_step, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 cache, bf16" if inp.dtype == "fp8" else inp.compute_dtype,
        "data": "synthetic (seeded; DeepSeek-V2 shapes, random-init weights)",
        "config": {
            "workload": inp.name, "batch": B, "seq_len": L, "heads": inp.dims.num_heads,
            "d_latent": inp.dims.d_latent, "d_rope": inp.dims.d_rope, "layout": inp.layout,
            "splits": S, "cache_copies_rotated": nbuf, "launch": "eager" if args.eager else "hip-graph",
            "parallelism": "single GPU",
        },
        "cache_GBps": round(gbps_step, 1),
        "cache_GBps_frac_of_8TBps": round(gbps_step / HBM_PEAK_GBPS, 4),
        "merge_out_proj_us": round(ms_rest * 1e3, 3),
        "merge_out_proj_fused": bool(pipe.fused),
        "roofline": {
            "kernel": "mla_decode",
            "bound": "hbm",
            "achieved": round(gbps_dec, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps_dec / HBM_PEAK_GBPS, 4),
            "achievable_read_GBps": round(probe_gbps, 1),
            "frac_of_measured": round(gbps_dec / probe_gbps, 4),
            "achievable_read_probe": "mla_read_probe: streaming 16-byte nontemporal loads over a 1 GiB buffer, "
                                     "20 back-to-back launches between two events",
            # the byte-counter profiles run each workload at the library's split count
            "traffic": hbm_traffic(inp.name) if not args.splits else None,
            "us_per_launch": round(ms_dec * 1e3, 3),
            "us_per_launch_p10_p50_p90": [round(dec_pct[q] * 1e3, 3) for q in (10, 50, 90)],
            "timing": "event pair carried by each decode launch (hipExtLaunchKernel) within whole steps",
            "algorithmic_bytes_per_launch": cache_bytes,
            "mfma_tflops": round(flops_dec / (ms_dec * 1e-3) / 1e12, 1),
            "mfma_frac_of_bf16_dense_peak": round(flops_dec / (ms_dec * 1e-3) / 2.5e15, 4),
        },
    }
    if inp.dims.hidden == 5120 and not args.eager:
        result["cache_append"] = cache_append_time(inp, stream)
        result["o_proj"] = o_proj_time(inp, stream)
        result["query_proj"] = query_proj_time(inp, stream)
        if inp.dtype == "bf16" and inp.name == "dsv2_b32_l4096":
            result["multi_token"] = multi_token_time(pipe, caches, stream)
            result["prefill"] = prefill_time(pipe, stream)
            result["layer"] = layer_time(inp, pipe, caches, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
