#!/usr/bin/env python3
"""Benchmark one MLA absorbed-decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

`--workload prefill_b4_s4k` measures the MHA-form prefill instead (a step
is mla_prefill_expand + mla_prefill_attn; value in TFLOP/s), and
`--workload out_fused_dsv3_m64` (or `_m128`) the output-side absorption
(a step is one mla_out_proj_fused call through the pre-fused W_O W_UV;
value in GB/s of the fused weight stream).

A step is the whole hot path on one batch of synthetic inputs already
resident in GPU memory: mla_absorb_q (W_UK absorption + query RoPE),
mla_decode_attn (split-K attention over the shared latent cache) and
mla_combine_out_proj (log-sum-exp merge and W_UV projection in one kernel),
all on one stream.
The default workload is DeepSeek-V3 shaped: batch 64, 8192 cached tokens per
sequence, 128 heads, latent 512 + RoPE 64, bf16, paged in 64-token blocks.

After the --warmup steps a settle phase of sustained steps (--settle-ms,
default 300 ms, reported as settle_ms) lets the GPU clock reach its steady
level; a timed region inside the clock ramp reads up to ~25% slower.  The
timed steps rotate over copies of the inputs (one per model layer, enough of
them to exceed the 256 MB Infinity Cache three times), each step one HIP
graph replay with its own events; ms_per_step is the median step.

Prints one JSON line on stdout.  `value` is cache GB/s of the whole step
(cached bytes / step time); `ms_per_step` gives the step latency.  The
`roofline` object rates the decode kernel alone, timed with HIP events on
the stream it runs on.  `cpu_baseline` times the float64 CPU oracle on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
INFINITY_CACHE_BYTES = 256 * 2**20
METRIC = "MLA decode µs/step, TFLOP/s and cache GB/s at B=64,L=8k,128 heads (% roofline)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def accounting(inp):
    """Algorithmic bytes and flops of one step (and of the decode kernel)."""
    c = inp.cfg
    tokens = int(inp.seq_lens.astype(np.int64).sum())
    B, Lq, H = c.batch, c.q_len, c.heads
    el = 4 if c.q_dtype == "f32" else 2
    cache = tokens * c.storage_bytes_per_token()
    w = (H * c.d_nope * c.d_latent + H * c.d_v * c.d_latent) * el
    q = B * Lq * H * (c.d_nope + c.d_rope) * el
    o = B * Lq * H * c.d_v * el
    attn_flops = 2.0 * H * Lq * tokens * (c.d_latent + c.d_rope + c.d_latent)
    proj_flops = 2.0 * B * Lq * H * (c.d_nope * c.d_latent + c.d_latent * c.d_v)
    return dict(tokens=tokens, cache_bytes=cache, step_bytes=cache + w + q + o,
                attn_flops=attn_flops, step_flops=attn_flops + proj_flops)


def clone_inputs(run_args: dict) -> dict:
    """A device copy of a step's inputs (a further layer): the cache pool,
    weights and queries are duplicated; the latent and RoPE views keep their
    offsets into the copied pool; sizes and scalars are shared."""
    out = dict(run_args)
    lat, rop = run_args["latent"], run_args["rope"]
    pool = lat.as_strided((lat.untyped_storage().nbytes() // lat.element_size(),), (1,), 0)
    pool2 = pool.clone()
    out["latent"] = pool2.as_strided(lat.shape, lat.stride(), lat.storage_offset())
    out["rope"] = pool2.as_strided(rop.shape, rop.stride(), rop.storage_offset())
    for k in ("q_nope", "q_rope", "w_uk", "w_uv", "kv_scale"):
        if run_args[k] is not None:
            out[k] = run_args[k].clone()
    return out


def cpu_baseline(inp, seconds: float):
    """Time the float64 oracle on a sample of (b, i, h) rows of the workload.

    One oracle call has a fixed cost (weights and the sampled sequences'
    cache converted to float64) and a cost per query row (that head's keys
    and values materialised over the whole sequence).  Calls on 1 and 8 rows
    estimate both; the timed call then takes as many rows as fill `seconds`.
    The value is the sample's share of the step's cache bytes over its time.
    """
    from threadpoolctl import threadpool_info

    from oracle import mla_decode

    c = inp.cfg
    rows_all = [(b, i, h) for b in range(c.batch) for i in range(c.q_len) for h in range(c.heads)]

    def timed(rows):
        t0 = time.perf_counter()
        mla_decode(inp, rows=rows)
        return time.perf_counter() - t0

    t1 = timed(rows_all[:1])
    t8 = timed(rows_all[:8])
    per_row = max((t8 - t1) / 7.0, 1e-4)
    fixed = max(t1 - per_row, 0.0)
    n = int(max(1, min(len(rows_all), (seconds - fixed) / per_row)))
    sample = rows_all[:n]
    dt = timed(sample)
    acc = accounting(inp)
    frac = n / len(rows_all)
    blas = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    cores = len(os.sched_getaffinity(0))
    seqs = sorted(set(r[0] for r in sample))
    return {"value": round(frac * acc["cache_bytes"] / dt / 1e9, 4), "unit": "GB/s",
            "cores": int(min(blas, cores)), "host_cpus": cores, "os_cpu_count": os.cpu_count(),
            "blas_threads": int(blas), "kind": "oracle",
            "sample": f"{n} of {len(rows_all)} (b,i,h) query rows (sequences {seqs[0]}..{seqs[-1]}), "
                      f"{dt:.1f} s; value = the sample's share of the step's cache bytes / time"}


def append_pass(mla, stream, n_tok: int, d_model: int, flush, reps: int) -> dict:
    """Time the cache-append producer for the step's n_tok new tokens: events
    around each launch, with a full decode step (604 MB of cache streamed at
    the headline) between launches so that its weights come from HBM, as
    they would between the layers of a model."""
    import torch

    from mla_inputs import AppendInputs

    inp = AppendInputs(n_tok, d_model, seed=20261211)
    dev = torch.device("cuda")

    def t(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(dt)

    h, wd, wr, wn = (t(a.view(np.int16), torch.bfloat16)
                     for a in (inp.h, inp.w_dkv, inp.w_kr, inp.kv_norm_w))
    pos = torch.from_numpy(inp.positions).to(dev)
    rows = torch.from_numpy(inp.rows).to(dev)
    pool = torch.empty((inp.pool_rows, 576), dtype=torch.bfloat16, device=dev)
    d = mla.append_dims(n_tok, d_model)
    ws = torch.empty(mla.mla_kv_append_workspace_bytes(d) // 4, dtype=torch.float32, device=dev)

    def run():
        mla.mla_kv_append(d, h, wd, wn, wr, pos, 10000.0, 1e-6, rows, pool,
                          pool.view(-1)[512:].data_ptr(), 576, None, ws, stream)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    run()
    for a, b in ev:
        flush()
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    nbytes = (576 * d_model + 512) * 2 + n_tok * d_model * 2 + n_tok * (576 * 2 + 4 + 8)
    flops = 2.0 * n_tok * 576 * d_model
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "tokens": n_tok, "d_model": d_model, "bytes": nbytes,
            "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 4), "tflops": round(flops / (us * 1e-6) / 1e12, 2),
            "kernels": "kv_down_kernel + kv_finish_kernel"}


def prefill_accounting(inp):
    """Flops of the MHA-form prefill: the expand GEMM over every cached token
    (H x (d_nope + d_v) outputs of width d_latent) and the causal attention
    (scores over d_nope + d_rope, values over d_v, visible pairs only)."""
    c = inp.cfg
    tokens = int(inp.seq_lens.astype(np.int64).sum())
    expand = 2.0 * tokens * c.d_latent * c.heads * (c.d_nope + c.d_v)
    pairs = 0
    for b in range(c.batch):
        n = int(inp.seq_lens[b])
        vis = np.arange(c.q_len) + n - c.q_len + 1 if c.causal else np.full(c.q_len, n)
        pairs += int(np.clip(vis, 0, n).sum())
    attn = 2.0 * c.heads * pairs * (c.d_nope + c.d_rope + c.d_v)
    return dict(tokens=tokens, expand_flops=expand, attn_flops=attn, pairs=pairs)


def prefill_main(args, name, torch):
    """One MHA-form prefill (mla_prefill_expand + mla_prefill_attn) of the
    prompt workload; a step is both calls.  Prints one JSON line."""
    import mla_latent_kv_lat_amd as mla
    from mla_inputs import PREFILL_CONFIGS, MLAInputs
    from mla_inputs.device import to_device

    cfg = PREFILL_CONFIGS[name]
    t0 = time.perf_counter()
    inp = MLAInputs(cfg)
    dev = to_device(inp)
    torch.cuda.synchronize()
    log(f"[bench] inputs for {name} ready in {time.perf_counter() - t0:.1f} s")
    d = mla.dims(cfg.batch, cfg.q_len, cfg.heads, cfg.d_nope, cfg.d_rope, cfg.d_latent, cfg.d_v,
                 mla.BF16, mla.BF16)
    T = dev.max_seq_len
    k_nope = torch.empty((cfg.batch, T, cfg.heads, cfg.d_nope), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((cfg.batch, T, cfg.heads, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((cfg.batch, cfg.q_len, cfg.heads, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((cfg.batch, cfg.q_len, cfg.heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def expand():
        mla.mla_prefill_expand(d, dev.latent, dev.kv_row_stride, dev.seq_lens, dev.block_table,
                               dev.max_blocks_per_seq, mla.TILE_TOKENS, T, dev.w_uk, dev.w_uv,
                               k_nope, v, stream)

    def attn():
        mla.mla_prefill_attn(d, dev.q_nope, dev.q_rope, dev.positions, dev.rope_base, k_nope, v,
                             dev.rope, dev.kv_row_stride, dev.seq_lens, dev.block_table,
                             dev.max_blocks_per_seq, mla.TILE_TOKENS, T, dev.causal,
                             dev.softmax_scale, o, lse, stream)

    for _ in range(args.warmup):
        expand()
        attn()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        expand()
        attn()
        settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    if not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite prefill output")

    # timed region: K steps, events around each call on the stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        ev[k][0].record(stream)
        expand()
        ev[k][1].record(stream)
        attn()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    ex_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    at_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in ev])
    ms = float(np.median(step_ms))
    acc = prefill_accounting(inp)
    flops = acc["expand_flops"] + acc["attn_flops"]
    at_med = float(np.median(at_ms))
    ex_med = float(np.median(ex_ms))
    tflops = flops / (ms * 1e-3) / 1e12
    at_tf = acc["attn_flops"] / (at_med * 1e-3) / 1e12
    ex_tf = acc["expand_flops"] / (ex_med * 1e-3) / 1e12
    traffic = None
    tpath = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                         "prefill_attn_b4_s4k_counters.json")
    if os.path.exists(tpath):
        try:
            with open(tpath) as f:
                tr = json.load(f)
            from mla_latent_kv_lat_amd.build import PREFILL_SOURCES, source_digest
            if tr.get("source_digest") == source_digest(PREFILL_SOURCES) and tr.get("workload") == name:
                traffic = tr.get("hbm_bytes_per_launch")
        except Exception as e:  # a stale or unreadable summary just leaves traffic unknown
            log(f"[bench] traffic summary not used: {e}")
    out = {
        "metric": f"MLA prefill (MHA form) TFLOP/s at B={cfg.batch}, S={cfg.q_len}, {cfg.heads} heads",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps,
        "pct_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": cfg.batch, "prompt_tokens": cfg.q_len,
                   "seq_len": cfg.max_seq_len, "heads": cfg.heads, "d_nope": cfg.d_nope,
                   "d_rope": cfg.d_rope, "d_latent": cfg.d_latent, "d_v": cfg.d_v,
                   "causal": bool(cfg.causal), "paged_block": 64 if cfg.paged else None,
                   "parallelism": "single GPU",
                   "flops": {"expand": acc["expand_flops"], "attention": acc["attn_flops"]}},
        "kernels_us": {"prefill_expand": round(ex_med * 1e3, 1), "prefill_attn": round(at_med * 1e3, 1),
                       "expand_tflops": round(ex_tf, 1),
                       "timing": "median of events around each call"},
        "roofline": {"bound": "mfma", "achieved": round(at_tf, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(at_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "prefill_attn_kernel", "launch_us": round(at_med * 1e3, 1),
                     "timing": "median of events around each launch, on its stream"},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = prefill_cpu_baseline(inp, acc, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def prefill_cpu_baseline(inp, acc, seconds: float):
    """The float64 oracle (the non-absorbed definition) on whole (sequence,
    head) pairs of the prefill: every query of one head of one prompt, which
    materialises that head's keys and values once, as the prefill does.
    value = the sample's share of the prefill's flops per second (all
    prompts have one length, so a pair's share is 1 / (B * H))."""
    from threadpoolctl import threadpool_info

    from oracle import mla_decode

    c = inp.cfg
    rng = np.random.default_rng(1)
    pairs = [(int(rng.integers(0, c.batch)), int(rng.integers(0, c.heads))) for _ in range(64)]

    def rows_of(ps):
        return [(b, i, h) for b, h in ps for i in range(c.q_len)]

    t1 = time.perf_counter()
    mla_decode(inp, rows=rows_of(pairs[:1]))
    per = max(time.perf_counter() - t1, 1e-3)
    n = int(max(1, min(len(pairs), seconds / per)))
    t1 = time.perf_counter()
    mla_decode(inp, rows=rows_of(pairs[:n]))
    dt = time.perf_counter() - t1
    frac = n / (c.batch * c.heads)
    blas = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    cores = len(os.sched_getaffinity(0))
    return {"value": round(frac * (acc["expand_flops"] + acc["attn_flops"]) / dt / 1e12, 6),
            "unit": "TFLOP/s", "cores": int(min(blas, cores)), "host_cpus": cores,
            "os_cpu_count": os.cpu_count(), "blas_threads": int(blas), "kind": "oracle",
            "sample": f"all {c.q_len} queries of {n} random (sequence, head) pairs of "
                      f"{c.batch * c.heads}, {dt:.1f} s (includes the oracle's float64 "
                      "conversion of its inputs); value = the sample's share of the prefill flops / time"}


def out_fused_main(args, name, torch):
    """The projection of one decode step's latent outputs through the
    pre-fused output weight (mla_out_proj_fused); a step is one call.  The
    unfused alternative's W_O product (a plain library GEMM on the W_UV
    outputs) is timed beside it for comparison.  Prints one JSON line."""
    import mla_latent_kv_lat_amd as mla
    from mla_inputs import OUT_FUSED_CONFIGS, OutProjInputs

    c = OUT_FUSED_CONFIGS[name]
    t0 = time.perf_counter()
    inp = OutProjInputs(c["m"], c["heads"], c["d_model"], seed=c["seed"], d_v=c["d_v"])
    M, H, dm, dv, dc = inp.m, inp.heads, inp.d_model, inp.d_v, inp.d_latent

    def dev(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()

    o_lat, w_o, w_uv = dev(inp.o_lat), dev(inp.w_o), dev(inp.w_uv)
    d = mla.dims(M, 1, H, 128, 64, dc, dv, mla.BF16, mla.BF16)
    stream = torch.cuda.current_stream()
    w_f = torch.empty((mla.mla_fused_out_weight_bytes(d, dm) // 2,), dtype=torch.bfloat16,
                      device="cuda")
    mla.mla_fuse_out_weight(d, dm, w_o, w_uv, w_f, stream)
    ws = torch.empty(mla.mla_out_proj_fused_workspace_bytes(d, dm) // 4, dtype=torch.float32,
                     device="cuda")
    out = torch.empty((M, dm), dtype=torch.bfloat16, device="cuda")
    # the unfused path's W_O product: o [M, H d_v] (the W_UV outputs) times W_O^T
    o_v = torch.randn((M, H * dv), dtype=torch.bfloat16, device="cuda")
    w_o_t = w_o.t().contiguous()
    out_u = torch.empty((M, dm), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] inputs for {name} ready in {time.perf_counter() - t0:.1f} s")

    def fused():
        mla.mla_out_proj_fused(d, dm, o_lat, w_f, ws, out, stream)

    def unfused():
        torch.mm(o_v, w_o_t, out=out_u)

    for _ in range(args.warmup):
        fused()
        unfused()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            fused()
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite fused output projection")

    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    f_ms = timed(fused)
    u_ms = timed(unfused)
    ms = float(np.median(f_ms))
    w_bytes = dm * H * dc * 2
    nbytes = w_bytes + M * H * dc * 2 + M * dm * 2
    flops = 2.0 * M * dm * H * dc
    gbs = nbytes / (ms * 1e-3) / 1e9
    u_bytes = dm * H * dv * 2 + M * H * dv * 2 + M * dm * 2
    u_us = float(np.median(u_ms)) * 1e3
    traffic = None
    tpath = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                         f"{name}_counters.json")
    if os.path.exists(tpath):
        try:
            with open(tpath) as f:
                tr = json.load(f)
            from mla_latent_kv_lat_amd.build import OUT_FUSED_SOURCES, source_digest
            if tr.get("source_digest") == source_digest(OUT_FUSED_SOURCES) and tr.get("workload") == name:
                traffic = tr.get("hbm_bytes_per_call")
        except Exception as e:  # a stale or unreadable summary just leaves traffic unknown
            log(f"[bench] traffic summary not used: {e}")
    out_line = {
        "metric": f"MLA fused output projection GB/s (pre-fused W_O W_UV, {H} heads, hidden {dm}, "
                  f"{M} query tokens)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps,
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "query_tokens": M, "heads": H, "d_latent": dc, "d_v": dv,
                   "d_model": dm, "fused_weight_MB": round(w_bytes / 1e6, 1),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "pack_rows_kernel + out_fused_kernel + out_sum_kernel",
                     "launch_us": round(ms * 1e3, 2),
                     "timing": "median of events around each call (its three kernels), on its stream"},
        "unfused_w_o_gemm": {"us": round(u_us, 2), "bytes": u_bytes,
                             "achieved_gbs": round(u_bytes / (u_us * 1e-6) / 1e9, 1),
                             "what": "torch.mm of the W_UV outputs [M, H d_v] by W_O^T (the unfused "
                                     "path's second product; its W_UV product is part of the fused "
                                     "combine kernel)"},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        out_line["cpu_baseline"] = out_fused_cpu_baseline(inp, nbytes, args.cpu_seconds)
    print(json.dumps(out_line), flush=True)


def out_fused_cpu_baseline(inp, nbytes: int, seconds: float):
    """The float64 oracle's fused projection (out_proj_fused) for a sample of
    output features: their fused-weight rows come from the oracle's
    fuse_out_weight (load time, untimed).  value = the sample's share of the
    call's bytes per second."""
    from threadpoolctl import threadpool_info

    from oracle import bf16_to_f64, fuse_out_weight, out_proj_fused

    rng = np.random.default_rng(2)
    o = bf16_to_f64(inp.o_lat)
    w_uv = bf16_to_f64(inp.w_uv)

    def fused_rows(k):
        ns = rng.choice(inp.d_model, k, replace=False)
        return fuse_out_weight(bf16_to_f64(inp.w_o[ns]), w_uv, inp.heads)

    def timed(wf):
        t1 = time.perf_counter()
        out_proj_fused(o, wf)
        return time.perf_counter() - t1

    # at most 1024 features: their fused rows alone are 0.5 GB of float64
    per = max(timed(fused_rows(16)) / 16, 1e-5)
    n = int(max(16, min(inp.d_model, 1024, seconds / per)))
    wf = fused_rows(n)
    # the oracle's product is one BLAS call: repeat it for a stable time
    reps, dt = 0, 0.0
    while reps == 0 or (dt < min(seconds, 3.0) and reps < 1000):
        dt += timed(wf)
        reps += 1
    dt /= reps
    blas = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    cores = len(os.sched_getaffinity(0))
    return {"value": round(n / inp.d_model * nbytes / dt / 1e9, 4), "unit": "GB/s",
            "cores": int(min(blas, cores)), "host_cpus": cores, "os_cpu_count": os.cpu_count(),
            "blas_threads": int(blas), "kind": "oracle",
            "sample": f"{n} of {inp.d_model} output features for all {inp.m} query tokens, "
                      f"{dt:.3f} s per call (mean of {reps}); value = the sample's share of the "
                      "call's bytes / time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU clock takes ~100 ms of sustained load to reach its steady
    # level; the settle phase after the warmup covers that whatever --warmup
    # says, so the timed steps measure the sustained rate of a decode loop
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--append-d-model", type=int, default=7168,
                    help="hidden width of the cache-append producer timed beside the step")
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed sustained steps after the warmup, so the clock is steady")
    ap.add_argument("--layer-copies", type=int, default=0,
                    help="input copies the steps rotate over (0: enough to exceed 3x the "
                         "256 MB Infinity Cache)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the one-GPU path only (asked for {max(args.gpus, world)} GPUs); "
              "the library runs the decode step on a single GPU (no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 1 << 28                                   # 2^28 float32 = 1 GiB
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}))
        return

    import mla_latent_kv_lat_amd as mla
    from mla_inputs import CONFIGS, HEADLINE, OUT_FUSED_CONFIGS, PREFILL_CONFIGS, MLAInputs
    from mla_inputs.device import to_device

    name = args.workload or HEADLINE
    if name in PREFILL_CONFIGS:
        prefill_main(args, name, torch)
        return
    if name in OUT_FUSED_CONFIGS:
        out_fused_main(args, name, torch)
        return
    cfg = CONFIGS[name]
    t0 = time.perf_counter()
    inp = MLAInputs(cfg)
    dev = to_device(inp)
    torch.cuda.synchronize()
    log(f"[bench] inputs for {name} ready in {time.perf_counter() - t0:.1f} s")

    DT = {"f32": mla.F32, "bf16": mla.BF16, "fp8": mla.FP8_E4M3}
    d = mla.dims(cfg.batch, cfg.q_len, cfg.heads, cfg.d_nope, cfg.d_rope, cfg.d_latent, cfg.d_v,
                 DT[cfg.q_dtype], DT[cfg.kv_dtype])
    step = mla.DecodeStep(d, num_splits=args.num_splits or None, keep_o_lat=False)
    G = step.num_splits
    stream = torch.cuda.current_stream()

    args_run = dict(q_nope=dev.q_nope, q_rope=dev.q_rope, positions=dev.positions, w_uk=dev.w_uk,
                    w_uv=dev.w_uv, latent=dev.latent, rope=dev.rope,
                    kv_row_stride=dev.kv_row_stride, kv_scale=dev.kv_scale,
                    seq_lens=dev.seq_lens, block_table=dev.block_table,
                    max_blocks_per_seq=dev.max_blocks_per_seq, max_seq_len=dev.max_seq_len,
                    causal=dev.causal, softmax_scale=dev.softmax_scale, rope_base=dev.rope_base)

    # ---- layer copies: the step's inputs (cache, weights, queries) are
    # replicated and the timed steps rotate over them, as the layers of a
    # model would, so that the working set of consecutive steps exceeds the
    # 256 MB Infinity Cache at least three times over and steps are served
    # from HBM, not from a cache that still holds the previous step's bytes
    acc0 = accounting(inp)
    part_bytes = step.o_part.numel() * step.o_part.element_size() + \
        step.q_abs.numel() * step.q_abs.element_size()
    ws_bytes = acc0["step_bytes"] + part_bytes
    n_copies = max(1, -(-3 * INFINITY_CACHE_BYTES // ws_bytes)) if args.layer_copies <= 0 \
        else args.layer_copies
    copies = [args_run] + [clone_inputs(args_run) for _ in range(n_copies - 1)]
    torch.cuda.synchronize()

    def run_copy(i):
        step.run(**copies[i % n_copies])

    # ---- warmup: the W steps asked for, then a settle phase of at least
    # --settle-ms of sustained steps: the GPU clock needs ~0.1 s of load to
    # reach its steady level, and a timed region inside the ramp reads up to
    # 25% slow.  Both are untimed; the line reports the settle phase.
    for i in range(args.warmup):
        run_copy(i)
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            run_copy(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    if not torch.isfinite(step.o.float()).all():
        raise RuntimeError("non-finite decode output")

    def timed_each(fn, k):
        """Events on the stream before and after each of k calls: per-call
        durations in ms and the whole region's."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(k):
            fn(i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        each = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(k)])
        return each, ev[0].elapsed_time(ev[k])

    # ---- eager launches, then the same steps replayed from HIP graphs (one
    # per layer copy, one step each), which skip the host launch overhead
    eager_each, _ = timed_each(run_copy, args.steps)
    graphs = [step.capture(steps=1, **c) for c in copies]
    t_settle = time.perf_counter()
    i = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms / 2:
        for _ in range(20):
            graphs[i % n_copies].replay()
            i += 1
        torch.cuda.synchronize()
    # ---- timed region: exactly K steps, one graph replay each, bracketed by
    # synchronisations; ms_per_step is the median step (the mean beside it)
    step_each, region_ms = timed_each(lambda i: graphs[i % n_copies].replay(), args.steps)
    ms_step = float(np.median(step_each))
    step_pct = [round(float(np.percentile(step_each, q)) * 1e3, 2) for q in (10, 50, 90)]

    # ---- per-kernel durations (events around each launch, same stream)
    def run_parts(i):
        c = copies[i % n_copies]
        return [lambda: mla.mla_absorb_q(d, c["q_nope"], c["q_rope"], c["positions"],
                                         c["rope_base"], c["w_uk"], step.q_abs, stream),
                lambda: mla.mla_decode_attn(d, step.q_abs, c["latent"], c["rope"],
                                            c["kv_row_stride"], c["kv_scale"], c["seq_lens"],
                                            c["block_table"], c["max_blocks_per_seq"],
                                            mla.TILE_TOKENS, c["max_seq_len"], c["causal"],
                                            c["softmax_scale"], G, step.o_part, step.lse_part,
                                            stream),
                lambda: mla.mla_combine_out_proj(d, G, c["seq_lens"], step.o_part, step.lse_part,
                                                 c["w_uv"], step.o, step.lse, None, stream)]

    n_parts = 3
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_parts)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        for f, (a, b) in zip(run_parts(k), evs[k]):
            a.record(stream)
            f()
            b.record(stream)
    torch.cuda.synchronize()
    kern_ms = [float(np.median([evs[k][j][0].elapsed_time(evs[k][j][1]) for k in range(args.steps)]))
               for j in range(n_parts)]

    kv_app = append_pass(mla, stream, cfg.batch * cfg.q_len, args.append_d_model,
                         lambda: step.run(**args_run), min(args.steps, 100))

    acc = acc0
    # bytes the rotation touches before a copy comes round again: below the
    # 256 MB Infinity Cache repeated steps would be served from it
    mall_hot = ws_bytes * n_copies < INFINITY_CACHE_BYTES
    us_step = ms_step * 1e3
    cache_gbs = acc["cache_bytes"] / (ms_step * 1e-3) / 1e9
    tflops = acc["step_flops"] / (ms_step * 1e-3) / 1e12
    t_roof = max(acc["step_flops"] / (PEAK_BF16_TFLOPS * 1e12), acc["step_bytes"] / (PEAK_HBM_GBS * 1e9))
    dec_s = kern_ms[1] * 1e-3
    dec_gbs = acc["cache_bytes"] / dec_s / 1e9
    dec_tflops = acc["attn_flops"] / dec_s / 1e12

    traffic = None
    util = None
    dec_kernel = "decode_sf_kernel<true>" if cfg.kv_dtype == "fp8" else "decode_sf_kernel<false>"
    tpath = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                         "decode_sf_b64_l8k_paged_counters.json")
    if os.path.exists(tpath):
        try:
            with open(tpath) as f:
                tr = json.load(f)
            from mla_latent_kv_lat_amd.build import DECODE_SOURCES, source_digest
            if (tr.get("source_digest") == source_digest(DECODE_SOURCES) and tr.get("workload") == name
                    and tr.get("kernel") == dec_kernel):
                traffic = tr.get("hbm_bytes_per_launch")
                util = tr.get("utilisation")
        except Exception as e:  # a stale or unreadable summary just leaves traffic unknown
            log(f"[bench] traffic summary not used: {e}")

    out = {
        "metric": METRIC,
        "value": round(cache_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(us_step, 2),
        "mean_us_per_step": round(region_ms / args.steps * 1e3, 2),
        "eager_us_per_step": round(float(np.median(eager_each)) * 1e3, 2),
        "step_us_p10_p50_p90": step_pct,
        "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps,
        "tflops": round(tflops, 2),
        "pct_roofline": round(100.0 * t_roof / (ms_step * 1e-3), 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.kv_dtype == "bf16" else ("fp8-cache/bf16" if cfg.kv_dtype == "fp8" else "f32"),
        "data": "synthetic",
        "config": {"workload": name, "batch": cfg.batch, "seq_len": cfg.max_seq_len,
                   "cached_tokens": acc["tokens"], "heads": cfg.heads, "q_len": cfg.q_len,
                   "d_latent": cfg.d_latent, "d_rope": cfg.d_rope, "d_nope": cfg.d_nope,
                   "d_v": cfg.d_v, "paged_block": 64 if cfg.paged else 0,
                   "kv_dtype": cfg.kv_dtype, "num_splits": G, "parallelism": "single GPU",
                   "working_set_MB": round(ws_bytes / 1e6, 1),
                   "layer_copies": n_copies,
                   "infinity_cache_hot": bool(mall_hot),
                   "launch": "HIP graph replay, one step of three kernels per replay, rotating over "
                             "the layer copies; median step (eager time beside)"},
        "kernels_us": {"absorb_q": round(kern_ms[0] * 1e3, 2), "decode_attn": round(kern_ms[1] * 1e3, 2),
                       "combine_out_proj": round(kern_ms[2] * 1e3, 2),
                       "timing": "events around each launch of eager steps (median)"},
        "kv_append": kv_app,
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": dec_kernel, "launch_us": round(kern_ms[1] * 1e3, 2),
                     "timing": "median of events around each decode launch of the eager steps, on its stream",
                     "mfma_tflops": round(dec_tflops, 1),
                     "mfma_frac": round(dec_tflops / PEAK_BF16_TFLOPS, 4),
                     "counters": util},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
