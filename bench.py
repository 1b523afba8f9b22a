#!/usr/bin/env python3
"""Throughput of one MLA decode step on one MI355X, as one JSON line.

A step is the whole hot path on one synthetic batch already resident in HBM:
  mla_absorb_q (q_nope . W_UK) -> mla_decode_paged (paged latent attention, split
  partitions + log-sum-exp combine) -> mla_out_proj (o_lat . W_UV).
Default workload: DeepSeek-V3-shaped bf16 decode, 64 sequences of 1024..8192 cached tokens
(uniform), 128 heads, d_c 512 + d_r 64, 64-token paged blocks in a shuffled block table, one
query token per sequence.  The other workloads (V2-Lite bf16, V3 with two query tokens, the
INT4 32K and INT2 128K caches, the tiny fp32 case) are selected with --workload.

value = cached-token.heads per second of step time, i.e. sum_b sum_i (L_b - s_q + i + 1) * H
divided by the mean step time.  Independent copies of the cache pool and of the weights are
rotated from step to step (and from call to call in the per-call timings), so the 256 MB
Infinity Cache cannot serve the cache or weight reads.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode cached-token·heads/s, HBM TB/s + MFMA util, µs/decode step"
UNIT = "cached-token·heads/s"
WORKLOADS = {"tiny-f32": "1", "v2lite-bf16": "2", "v3-bf16-sq1": "3", "v3-bf16-sq2": "3b",
             "v2lite-int4-32k": "4", "v3-int2-128k": "5", "v3-gqa-sq2": "3b"}
# GQLA's per-group GQA path on the V3 batch with two query tokens: head groups sharing their
# key/value up-projections, the latent expanded per group
GQA_GROUPS = {"v3-gqa-sq2": 8}
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
KERNEL_SOURCES = ["mla_latent_kv_02_amd/csrc/mla_decode.hip", "mla_latent_kv_02_amd/csrc/mla_decode_rows.hip",
                  "mla_latent_kv_02_amd/csrc/mla_combine.hip", "mla_latent_kv_02_amd/csrc/mla_stage.hpp",
                  "mla_latent_kv_02_amd/csrc/mla_device.hpp", "mla_latent_kv_02_amd/csrc/mla_internal.hpp"]


GQA_KERNEL_SOURCES = ["mla_latent_kv_02_amd/csrc/mla_gqa.hip", "mla_latent_kv_02_amd/csrc/mla_combine.hip",
                      "mla_latent_kv_02_amd/csrc/mla_stage.hpp", "mla_latent_kv_02_amd/csrc/mla_device.hpp",
                      "mla_latent_kv_02_amd/csrc/mla_internal.hpp"]


def kernel_hash(sources=None) -> str:
    """Hash of the decode kernels' code: the sources with comments and layout removed, so that
    an edit of a comment keeps the counter summaries that were measured on the same code."""
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        text = open(os.path.join(ROOT, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counted_traffic(workload: str, sources=None):
    """Bytes per launch measured by the FETCH_SIZE / WRITE_SIZE counters for this workload, while
    the summary's kernel source hash matches the current sources; else None."""
    tfile = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.json")
    if os.path.exists(tfile):
        try:
            tr = json.load(open(tfile))
            if tr.get("kernel_hash") == kernel_hash(sources):
                return tr.get("bytes_per_launch")
        except Exception:
            pass
    return None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v3-bf16-sq1", choices=sorted(WORKLOADS))
    ap.add_argument("--num-splits", type=int, default=0, help="context partitions (0 = library plan)")
    ap.add_argument("--rotate", type=int, default=0, help="cache pool copies to rotate (0 = enough to exceed 512 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch", default="graph", choices=["graph", "step-graph", "eager"],
                    help="timed steps as one HIP graph of all K steps (default), one graph replay per "
                         "step, or eager launches")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--profile-run", action="store_true",
                    help="run warmup+steps and a 256 MiB copy for counter calibration; print no JSON")
    return ap.parse_args()


def algorithmic(x, bytes_per_token):
    """Bytes and FLOPs the decode (attention) step must move / compute, and the metric's units."""
    cfg = x.cfg
    L = x.seq_lens.astype("int64")
    H, s_q = cfg.H, cfg.s_q
    qbytes = 2 if cfg.dtype == "bf16" else 4
    cache_bytes = int(L.sum()) * bytes_per_token
    io_bytes = len(L) * s_q * H * ((cfg.d_c + cfg.d_r) * qbytes + cfg.d_c * 4 + 4)
    attended = sum(int((L - s_q + i + 1).sum()) for i in range(s_q))       # (query, token) pairs
    flops = attended * H * 2 * (2 * cfg.d_c + cfg.d_r)
    return cache_bytes + io_bytes, cache_bytes, flops, attended * H


def cpu_baseline(x, seconds: float):
    """Time the float64 oracle (the unabsorbed MLA definition) on a bounded sample of sequences."""
    import oracle
    cfg = x.cfg
    lens = [int(L) for L in x.seq_lens]
    if cfg.quantised:
        c, k = oracle.dequant_cache([x.c_codes[b, :L] for b, L in enumerate(lens)],
                                    [x.c_sz[b, :L] for b, L in enumerate(lens)],
                                    [x.r_codes[b, :L] for b, L in enumerate(lens)],
                                    [x.r_sz[b, :L] for b, L in enumerate(lens)], cfg.latent_group, cfg.rope_group)
    else:
        c = [x.c[b, :L] for b, L in enumerate(lens)]
        k = [x.k_rope[b, :L] for b, L in enumerate(lens)]
    done_units, t_used, nseq = 0, 0.0, 0
    order = list(range(len(x.seq_lens)))
    # sample: whole sequences (all heads, all query tokens) until ~`seconds` of CPU time
    for b in order * 1000:
        t0 = time.perf_counter()
        oracle.decode_unabsorbed(x.q_nope[b:b + 1], x.q_rope[b:b + 1], x.w_uk, x.w_uv, [c[b]], [k[b]],
                                 x.seq_lens[b:b + 1], cfg.s_q, cfg.sm_scale)
        t_used += time.perf_counter() - t0
        L = int(x.seq_lens[b])
        done_units += sum(L - cfg.s_q + i + 1 for i in range(cfg.s_q)) * cfg.H
        nseq += 1
        if t_used >= seconds:
            break
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    return {"value": done_units / t_used, "unit": UNIT, "cores": int(threads), "kind": "oracle",
            "sample": f"float64 unabsorbed oracle (explicit per-head K=[c W_UK^T | k_rope], V=c W_UV, softmax), "
                      f"{nseq} sequence passes over the batch of {len(x.seq_lens)}, all {cfg.H} heads; {t_used:.1f} s",
            "seconds": round(t_used, 2)}


def bench_gqa(args, x, cfg, G, dev):
    """GQLA's GQA decode path: the batch's latent expanded per group (mla_gqa_expand, group g
    taking head g's W_UK / W_UV), then grouped-query attention over the expanded cache
    (mla_gqa_decode_paged), timed like the MLA decode.  Output is already in value space."""
    import numpy as np
    import torch
    import mla_latent_kv_02_amd as mla
    B, s_q, H = len(x.seq_lens), cfg.s_q, cfg.H
    L = x.seq_lens
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(dev)  # noqa: E731
    w_uk_g, w_uv_g = bf(x.w_uk[:G]), bf(x.w_uv[:G])
    nb = x.pool.shape[0]
    bb = mla.gqa_block_bytes(G)
    rotate = args.rotate or max(2, math.ceil(512e6 / (nb * bb)) + 1)
    bt = torch.from_numpy(x.block_table).to(dev)
    sl = torch.from_numpy(L).to(dev)
    pos = np.concatenate([np.arange(Lb) for Lb in L])
    seq = np.repeat(np.arange(B), L)
    slots = torch.from_numpy((x.block_table[seq, pos // 64].astype("int64") * 64 + pos % 64).astype("int32")).to(dev)
    rows = bf(np.concatenate([x.c[b, :Lb] for b, Lb in enumerate(L)]))
    krows = bf(np.concatenate([x.k_rope[b, :Lb] for b, Lb in enumerate(L)]))
    pools = []
    for _ in range(rotate):
        gp = torch.zeros((nb, bb), dtype=torch.uint8, device=dev)
        mla.gqa_expand(rows, krows, w_uk_g, w_uv_g, gp, slots)
        pools.append(gp)
    torch.cuda.synchronize()
    del rows, krows
    qn, qr = bf(x.q_nope), bf(x.q_rope)
    max_len, total_len = int(L.max()), int(L.astype("int64").sum())
    out = torch.empty((B, s_q, H, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((B, s_q, H), dtype=torch.float32, device=dev)
    mla.gqa_decode_paged(qn, qr, pools[0], G, bt, sl, max_len, cfg.sm_scale, args.num_splits, out=out, lse=lse,
                         total_seq_len=total_len)
    a = mla._gqa_args(qn, qr, pools[0], G, bt, sl, max_len, cfg.sm_scale, args.num_splits, out, lse, None, total_len)
    import ctypes
    n = ctypes.c_size_t()
    mla._check(mla.lib().mla_gqa_workspace_size(ctypes.byref(a), ctypes.byref(n)), "mla_gqa_workspace_size")
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
    call = lambda i: mla.gqa_decode_paged(qn, qr, pools[i % rotate], G, bt, sl, max_len, cfg.sm_scale,  # noqa: E731
                                          args.num_splits, out=out, lse=lse, workspace=ws, total_seq_len=total_len)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    if args.profile_run:
        for i in range(args.steps):
            call(i)
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)          # calibration copy: 256 MiB read + 256 MiB written
        torch.cuda.synchronize()
        print(f"profile run done: {args.steps} calls of {args.workload}, 1 calibration copy of 256 MiB", flush=True)
        return None
    st = torch.cuda.current_stream(dev)
    reps = rotate * max(1, math.ceil(8 / rotate))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    K = args.steps
    replays = max(2, math.ceil(K / reps))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * reps)
    Ll = L.astype("int64")
    cache_bytes = int(Ll.sum()) * (G * 512 + 128)
    io_bytes = B * s_q * H * ((128 + 64) * 2 + 128 * 4 + 4)
    attended = sum(int((Ll - s_q + i + 1).sum()) for i in range(s_q))
    flops = attended * H * 2 * (192 + 128)
    units = attended * H
    gbs = (cache_bytes + io_bytes) / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "mla_gqa_decode_paged (gqa_decode_kernel + combine_kernel)",
            "algorithmic_bytes_per_launch": cache_bytes + io_bytes, "flops_per_launch": flops,
            "traffic": counted_traffic(args.workload, GQA_KERNEL_SOURCES)}
    return {"metric": METRIC, "value": units / (ms * 1e-3), "unit": UNIT, "n_gpus": 1, "steps": replays * reps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": args.workload, "batch": B, "heads": H, "groups": G, "s_q": s_q, "d_n": 128,
                       "d_v": 128, "d_r": 64, "cache": "bf16 per-group expanded",
                       "mean_seq_len": float(L.mean()), "block_tokens": 64, "pool_copies_rotated": rotate},
            "roofline": roof, "us_per_step": round(ms * 1e3, 2), "decode_us": round(ms * 1e3, 2),
            "step_launch": "hip_graph", "hbm_tbps": round(gbs / 1e3, 3), "cache_bytes": cache_bytes,
            "note": "a step is the GQA path's whole decode: no absorption or up-projection on this path"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the decode shards over sequences "
                                   "with no communication, so run one process per GPU instead",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    import mla_latent_kv_02_amd as mla
    from mla_synth import CONFIGS, SEEDS, make_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    mla.lib()
    name = WORKLOADS[args.workload]
    cfg = CONFIGS[name]
    dev = torch.device("cuda:0")
    log(f"generating {args.workload} inputs")
    x = make_inputs(cfg, SEEDS[name])
    log("inputs ready; uploading")
    if args.workload in GQA_GROUPS:
        rec = bench_gqa(args, x, cfg, GQA_GROUPS[args.workload], dev)
        if rec is None:
            return
        log(f"gqa decode {rec['decode_us']:.2f} us")
        print(json.dumps(rec), flush=True)
        return
    desc = mla.cache_desc(cfg.d_c, cfg.d_r, cfg.latent_fmt, cfg.rope_fmt, cfg.latent_group, cfg.rope_group)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    pool_bytes = x.pool.nbytes
    rotate = args.rotate or max(3, math.ceil(512e6 / pool_bytes) + 1)
    pools = [torch.from_numpy(x.pool).to(dev) for _ in range(rotate)]
    bt = torch.from_numpy(x.block_table).to(dev)
    sl = torch.from_numpy(x.seq_lens).to(dev)
    qn = torch.from_numpy(x.q_nope).to(dt).to(dev)
    qr = torch.from_numpy(x.q_rope).to(dt).to(dev)
    wuk = torch.from_numpy(x.w_uk).to(dt).to(dev)
    wuv = torch.from_numpy(x.w_uv).to(dt).to(dev)
    # weight copies: enough that a call cycling over them reads more than 512 MB before it
    # comes back to one (W_UK and W_UV of the V3 shapes are 16.8 MB each)
    w_bytes = wuk.numel() * wuk.element_size()
    n_w = max(rotate, min(256, math.ceil(512e6 / w_bytes) + 1))
    wuks = [wuk] + [wuk.clone() for _ in range(n_w - 1)]
    wuvs = [wuv] + [wuv.clone() for _ in range(n_w - 1)]
    max_len = int(x.seq_lens.max())
    total_len = int(x.seq_lens.astype("int64").sum())
    # one step object per rotated pool, each with its own weight copy
    steps = [mla.DecodeStep(wuks[i], wuvs[i], desc, len(x.seq_lens), cfg.s_q, max_len, cfg.sm_scale,
                            num_splits=args.num_splits, q_lat_dtype=dt, total_seq_len=total_len)
             for i in range(rotate)]
    step = steps[0]
    B, s_q, H = len(x.seq_lens), cfg.s_q, cfg.H
    ql = step.q_lat.view(B, s_q, H, cfg.d_c)

    for i in range(args.warmup):
        steps[i % rotate].run(qn, qr, pools[i % rotate], bt, sl)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps, {rotate} pool copies, {n_w} weight copies)")

    if args.profile_run:
        for i in range(args.steps):
            steps[i % rotate].run(qn, qr, pools[i % rotate], bt, sl)
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)          # calibration copy: 256 MiB read + 256 MiB written
        torch.cuda.synchronize()
        print(f"profile run done: {args.steps} steps of {args.workload}, 1 calibration copy of 256 MiB", flush=True)
        return

    K = args.steps
    st = torch.cuda.current_stream(dev)
    splits, tpc = mla.decode_plan(ql, qr, pools[0], desc, bt, sl, max_len, cfg.sm_scale, args.num_splits,
                                  total_seq_len=total_len)
    # (1) the step: absorb -> decode -> out_proj on the rotated cache pools.  Timed as one HIP
    # graph that holds all K steps (as a deployed decode graph holds every layer), replayed
    # once; one graph replay per step and eager launches are timed after it for the record.
    # On this runtime every graph launch leaves the GPU idle for a while at its boundary, and
    # eager launches are paced by the host's argument marshalling when its cores are slow.
    graphs = [steps[i].capture(qn, qr, pools[i], bt, sl) for i in range(rotate)]
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all):
        for i in range(K):
            steps[i % rotate].run(qn, qr, pools[i % rotate], bt, sl)

    def timed_steps(mode):
        def one(i):
            graphs[i % rotate].replay() if mode == "step-graph" else steps[i % rotate].run(qn, qr, pools[i % rotate], bt, sl)
        for i in range(args.warmup):
            one(i)
        if mode == "graph":
            g_all.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(st)
        if mode == "graph":
            g_all.replay()
        else:
            for i in range(K):
                one(i)
        e1.record(st)
        torch.cuda.synchronize()
        return max(e0.elapsed_time(e1) / K, 1e-9), time.perf_counter() - t0

    ms_per_step, wall = timed_steps(args.launch)
    mode_us = {m: round((ms_per_step if m == args.launch else timed_steps(m)[0]) * 1e3, 2)
               for m in ("graph", "step-graph", "eager")}
    # per-step spread: K more steps, one graph replay per step, each between its own pair of events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        evs[i][0].record(st)
        graphs[i % rotate].replay()
        evs[i][1].record(st)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    p10, p50, p90 = (float(v) for v in np.percentile(per_step, [10, 50, 90]))
    # (2) per-call durations: each library call is captured REPS times back to back in a HIP
    # graph (the decode cycling over the rotated pools) and the graph is replayed between two
    # events on this stream, so the figure is GPU time per call without host launch gaps
    def capture_calls(fn, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        return g

    def call_ms(g, reps, replays):
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(replays):
            g.replay()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (replays * reps)

    reps_dec = rotate * max(1, math.ceil(8 / rotate))
    g_abs = capture_calls(lambda i: mla.absorb_q(qn.view(B * s_q, H, cfg.d_n), wuks[i], out=step.q_lat), n_w)
    g_dec = capture_calls(lambda i: mla.decode_paged(ql, qr, pools[i % rotate], desc, bt, sl, max_len, cfg.sm_scale,
                                                     args.num_splits, out=step.o_lat, lse=step.lse,
                                                     workspace=step.workspace, total_seq_len=total_len), reps_dec)
    g_out = capture_calls(lambda i: mla.out_proj(step.o_lat.view(B * s_q, H, cfg.d_c), wuvs[i], out=step.out), n_w)
    replays = max(2, math.ceil(K / 8))
    absorb_ms = call_ms(g_abs, n_w, replays)
    decode_ms = call_ms(g_dec, reps_dec, replays)
    proj_ms = call_ms(g_out, n_w, replays)

    # (3) the cache writer for this step's new tokens (the last s_q positions of every
    # sequence), timed like the calls above after the decode timings, into one pool copy
    pos = (x.seq_lens.astype("int64")[:, None] - s_q + np.arange(s_q)[None, :]).reshape(-1)
    seq = np.repeat(np.arange(B), s_q)
    slots = torch.from_numpy((x.block_table[seq, pos // 64].astype("int64") * 64 + pos % 64).astype("int32")).to(dev)
    gen = torch.Generator(device=dev).manual_seed(1234)
    c_new = torch.randn((B * s_q, cfg.d_c), generator=gen, device=dev).to(qr.dtype)
    k_new = torch.randn((B * s_q, cfg.d_r), generator=gen, device=dev).to(qr.dtype)
    g_app = capture_calls(lambda i: mla.append_kv(c_new, k_new, pools[0], desc, slots), 8)
    append_ms = call_ms(g_app, 8, replays)
    # (4) quantised caches: the same decode with the history split by precision, a bf16 sink
    # of 64 tokens and a bf16 recent window of 512 around the workload's low-bit cache: as
    # three parts, and with sink and window in one bf16 cache (the recent part; attention
    # does not depend on token order apart from the causal mask at the end)
    mixed_ms = mixed2_ms = None
    if cfg.quantised:
        hi_desc = mla.cache_desc(cfg.d_c, cfg.d_r, "bf16")
        S, W = 64, 512
        hi_pool = torch.zeros((B * (1 + W // 64), mla.block_bytes(hi_desc)), dtype=torch.uint8, device=dev)
        hi_pool.view(torch.bfloat16).normal_(generator=gen)
        sink_bt = torch.arange(B, dtype=torch.int32, device=dev).view(B, 1)
        rec_bt = (B + torch.arange(B * (W // 64), dtype=torch.int32, device=dev)).view(B, W // 64)
        sink_l = torch.full((B,), S, dtype=torch.int32, device=dev)
        rec_l = torch.full((B,), W, dtype=torch.int32, device=dev)
        mid_l = (sl - S - W).clamp(min=0)
        g_mix = capture_calls(lambda i: mla.decode_mixed(
            ql, qr, (hi_pool, hi_desc, sink_bt, sink_l, S), (pools[i % rotate], desc, bt, mid_l, max_len),
            (hi_pool, hi_desc, rec_bt, rec_l, W), cfg.sm_scale), reps_dec)
        mixed_ms = call_ms(g_mix, reps_dec, replays)
        both_bt = (torch.arange(B * (1 + W // 64), dtype=torch.int32, device=dev)).view(B, 1 + W // 64)
        both_l = torch.full((B,), S + W, dtype=torch.int32, device=dev)
        g_mix2 = capture_calls(lambda i: mla.decode_mixed(
            ql, qr, None, (pools[i % rotate], desc, bt, mid_l, max_len), (hi_pool, hi_desc, both_bt, both_l, S + W),
            cfg.sm_scale), reps_dec)
        mixed2_ms = call_ms(g_mix2, reps_dec, replays)
    # (5) the fixed latent rotation folded into W_UK (an offline step), on a copy of W_UK
    wuk_copy = wuk.clone()
    g_rot = capture_calls(lambda i: mla.hadamard_rotate(wuk_copy, dim=2), 8)
    rotate_ms = call_ms(g_rot, 8, replays)
    rotate_gbs = 2 * wuk_copy.numel() * wuk_copy.element_size() / (rotate_ms * 1e-3) / 1e9

    bpt = mla.block_bytes(desc) // 64
    alg_bytes, cache_bytes, flops, units = algorithmic(x, bpt)
    value = units / (ms_per_step * 1e-3)
    dec_s = decode_ms * 1e-3
    gbs = alg_bytes / dec_s / 1e9
    tflops = flops / dec_s / 1e12
    ai = flops / alg_bytes
    bound = "hbm" if ai < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    if cfg.dtype != "bf16":
        roof["kernel"] = "mla_decode_paged (decode_f32_kernel + combine_kernel)"
    elif s_q * H >= 96:
        roof["kernel"] = "mla_decode_paged (decode_rows_kernel + combine_rows_kernel)"
    elif cfg.latent_fmt in ("int4", "int2") and s_q * H <= 16:
        roof["kernel"] = "mla_decode_paged (decode_pipe_kernel + combine_part_kernel)"
    else:
        roof["kernel"] = "mla_decode_paged (decode_mfma_kernel + combine_part_kernel)"
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    roof["flops_per_launch"] = flops
    roof["traffic"] = counted_traffic(args.workload)

    rec = {"metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
           "config": {"workload": args.workload, "batch": B, "heads": H, "s_q": s_q, "d_c": cfg.d_c,
                      "d_r": cfg.d_r, "d_n": cfg.d_n, "d_v": cfg.d_v, "cache": cfg.latent_fmt + "/" + cfg.rope_fmt,
                      "seq_len": cfg.lens[1] if cfg.lens[0] == "fixed" else list(cfg.lens[1:]),
                      "mean_seq_len": float(x.seq_lens.mean()), "block_tokens": 64, "splits": splits,
                      "tiles_per_split": tpc, "pool_copies_rotated": rotate, "weight_copies_rotated": n_w},
           "roofline": roof,
           "us_per_step": round(ms_per_step * 1e3, 2), "wall_us_per_step": round(wall / K * 1e6, 2),
           "step_graph_us_p10_p50_p90": [round(p10, 2), round(p50, 2), round(p90, 2)],
           "step_launch": {"graph": "one HIP graph of the K steps", "step-graph": "one HIP graph per step",
                           "eager": "eager launches"}[args.launch],
           "us_per_step_by_launch": mode_us,
           "call_timing": "per-call HIP graphs of back-to-back calls, events on the launch stream",
           "decode_us": round(decode_ms * 1e3, 2), "absorb_us": round(absorb_ms * 1e3, 2),
           "out_proj_us": round(proj_ms * 1e3, 2), "append_us": round(append_ms * 1e3, 2),
           "append_tokens": B * s_q, "rotate_w_uk_us": round(rotate_ms * 1e3, 2),
           "rotate_w_uk_gbs": round(rotate_gbs, 1),
           "mixed_decode_us": round(mixed_ms * 1e3, 2) if mixed_ms is not None else None,
           "mixed_decode_2part_us": round(mixed2_ms * 1e3, 2) if mixed2_ms is not None else None,
           "hbm_tbps": round(gbs / 1e3, 3),
           "mfma_util": round(tflops / BF16_PEAK_TFLOPS, 4), "cache_bytes": cache_bytes}
    log(f"timed {K} steps: {ms_per_step * 1e3:.2f} us/step, decode {decode_ms * 1e3:.2f} us")
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host")
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
