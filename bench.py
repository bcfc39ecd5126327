#!/usr/bin/env python3
"""LSA decode hot-path benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg4]

A bench step is one pass of the whole hot path: one lsa_step64 window.
That is 64 decode steps of lightning refine + top-k + sparse decode attention
for every request, plus the next window's chunk scoring, threshold
selection and slot-pool refill from the cold tier (pinned host memory,
hipMemcpyAsync on a side stream).  Inputs are seeded synthetic tensors
already resident in HBM / pinned memory when timing starts.

Prints one JSON line:
  value        decode steps per second (each decode step serves every request)
  roofline     for the kernel with the largest share of the window's time,
               algorithmic work per launch / its mean HIP-event duration
  cpu_baseline the CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSA decode steps/s + scoring/attn HBM GB/s (% of peak) at 128K and 500K ctx"
HBM_PEAK_GBS = 8000.0
# fp32 VALU fma without packed ops: 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz
VALU_F32_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
MFMA_BF16_PEAK_TFLOPS = 2500.0
# In the timed region every TIMING_EVERY-th launch of the dominant kernel is
# bracketed by HIP events (each record costs a few microseconds of GPU time).
TIMING_EVERY = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(name, cfg, inp, sel_cnt, k, tcnt_total, B):
    """Algorithmic bytes and flops of one launch of a kernel in one window."""
    eb = {0: 4, 1: 2, 2: 1}
    n_cand = int(sel_cnt.sum()) * cfg.chunk
    nrec = int(inp["n_rec"].sum())
    nh = int(inp["chunk_off"][-1])
    if name == "k_refine":
        per = cfg.d * eb[cfg.idx_dtype]
        flops = n_cand * (2 * cfg.H * cfg.d + 2 * cfg.H + 1)
        return n_cand * per + int(sel_cnt.sum()) * 4 + n_cand * 4, flops
    if name == "k_refine_mfma":
        # key rows of every candidate, its |key|^2 (formed once per window by
        # the pipeline), its (L, U) pair out, and the chunk's page + scale
        nsel = int(sel_cnt.sum())
        per = cfg.d * eb[cfg.idx_dtype] + 4 + 8
        return n_cand * per + nsel * (8 if cfg.idx_dtype == 2 else 4), n_cand * 2 * cfg.H * cfg.d
    if name == "k_key_norm2":
        # key rows of every candidate in, one fp32 norm per candidate out
        return n_cand * (cfg.d * eb[cfg.idx_dtype] + 4), n_cand * 2 * cfg.d
    if name in ("k_attn_mla", "k_attn_f32"):
        toks = tcnt_total + nrec
        row = cfg.Dk * eb[cfg.kv_dtype]
        qb = B * cfg.Hq * cfg.Dk * eb[cfg.kv_dtype]
        return toks * row + qb, toks * cfg.Hq * (cfg.Dk + cfg.Dv) * 2
    if name == "k_score":
        per = cfg.d * eb[cfg.idx_dtype] + (4 if cfg.idx_dtype == 2 else 0) + 4
        return nh * per, nh * 2 * cfg.d
    if name == "k_topk":
        return n_cand * 4 + B * k * 4, 0
    if name == "k_select":
        return nh * 4 + int(sel_cnt.sum()) * 4, 0
    return 0, 0


def traffic_for(kernel, workload, launches_per_window):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(workload, {}).get(kernel)
    from learned_sparse_kv_amd.profsum import KERNEL_SOURCE, source_hash
    if not e or kernel not in KERNEL_SOURCE or e.get("source_hash") != source_hash(KERNEL_SOURCE[kernel]):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(inp, cfg, threads, requests=None):
    """The oracle on one trigger (score + select) and one decode step (refine,
    top-k, attention) of the given requests (default: all)."""
    from oracle import oracle
    reqs = list(range(cfg.batch)) if requests is None else list(requests)
    o = oracle.Oracle(inp)
    t0 = time.perf_counter()
    _, sel, cnt = o.score_select()
    units = [(r, 0) for r in reqs]
    o.decode_units(units, sel, cnt, cfg.topk, cfg.sm_scale, threads=threads)
    dt = time.perf_counter() - t0
    frac = len(reqs) / cfg.batch  # share of one decode step of the whole batch
    return {"value": round(frac / dt, 4), "unit": "decode steps/s", "cores": threads,
            "kind": "oracle", "cpu": _cpu_model(),
            "sample": f"one trigger (score+select, all {cfg.batch} requests) and one decode step "
                      f"(refine+top-k+attention) of {len(reqs)} of the {cfg.batch} requests of "
                      f"{cfg.name}, scaled to whole-batch steps; {dt:.1f} s wall on {threads} "
                      f"thread(s)"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def hbm_calibration(nbytes=1 << 30, reps=5):
    """Plain device copy (read + write) and plain reduction (read) of a large
    buffer with torch, for the achievable-bandwidth line beside the kernels."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    y.copy_(x)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 1e3 / reps
    s = x.sum()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        s = x.sum()
    e1.record()
    torch.cuda.synchronize()
    read_s = e0.elapsed_time(e1) / 1e3 / reps
    # the library's plain streaming-read kernel: the achievable-read line
    from learned_sparse_kv_amd import lsa
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lsa.lsa_stream_read(x, nbytes, sink)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        lsa.lsa_stream_read(x, nbytes, sink)
    e1.record()
    torch.cuda.synchronize()
    stream_s = e0.elapsed_time(e1) / 1e3 / reps
    del x, y, sink
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "copy_gbs": round(2 * nbytes / copy_s / 1e9, 1),
            "torch_sum_read_gbs": round(nbytes / read_s / 1e9, 1),
            "stream_read_gbs": round(nbytes / stream_s / 1e9, 1)}


def sustained_scoring(label, B, L, idx_dt, H=64, d=128, window=8192, seed=0, reps=3, layers=1,
                      sigmoid=False, theta=0.5):
    """lsa_score_chunks + lsa_select_threshold over many distinct KIComp buffers
    (together more than twice the 256 MB last-level cache), so every launch
    streams cold lines: B requests of L tokens each, one launch per trigger.
    layers > 1: the OR-mode union over that many indexer layers
    (lsa_score_chunks_union), each layer reading its own buffer.
    sigmoid: the per-head sigmoid score (lsa_score_chunks_sigmoid) with the
    0.5 threshold; its bound is fp32 vector arithmetic (H*d fma per chunk)."""
    import math
    import numpy as np
    import torch
    from learned_sparse_kv_amd import lsa, synth
    g = lsa.Geom(np.full(B, L, np.int32), window)
    nhist = (max(L - window, 0) // 64)
    nh = B * nhist
    row = d * (1 if idx_dt == synth.FP8 else 2)
    per = nh * (row + (4 if idx_dt == synth.FP8 else 0))  # algorithmic bytes per trigger
    nbuf = max(6, math.ceil(600e6 / per))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    kic, ksc = [], []
    for _ in range(nbuf):
        x = torch.randn(nh, d, generator=gen, device="cuda") * (d ** -0.5)
        if idx_dt == synth.FP8:
            kic.append((x * 448.0 / 4.0).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8))
            ksc.append(torch.full((nh,), 4.0 / 448.0, device="cuda"))
        else:
            kic.append(x.to(torch.bfloat16).view(torch.int16))
            ksc.append(None)
        del x
    qs = [(torch.randn(B, H, d, generator=gen, device="cuda") * (H / 4) ** 0.5).to(torch.bfloat16).view(torch.int16)
          for _ in range(layers)]
    q = qs[0]
    w = torch.full((B, H), 1.0 / H, device="cuda")
    bias = torch.full((B,), -1.0, device="cuda")
    z = torch.empty(nh, device="cuda")
    sel = torch.empty(nh, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(lsa.lsa_score_ws_bytes(g, d), 256), dtype=torch.uint8, device="cuda")

    def trig(b):
        if sigmoid:
            lsa.lsa_score_chunks_sigmoid(g, q, synth.BF16, w, bias, theta, H, d, kic[b], idx_dt, ksc[b], z)
            lsa.lsa_select_threshold(g, z, theta, sel, cnt)
            return
        if layers == 1:
            lsa.lsa_score_chunks(g, q, synth.BF16, w, bias, H, d, kic[b], idx_dt, ksc[b], z, ws)
        else:
            bs = [(b + l) % nbuf for l in range(layers)]
            lsa.lsa_score_chunks_union(g, qs, synth.BF16, [w] * layers, [bias] * layers, H, d,
                                       [kic[x] for x in bs], idx_dt, [ksc[x] for x in bs], z, ws)
        lsa.lsa_select_threshold(g, z, 0.0, sel, cnt)

    for b in range(nbuf):
        trig(b)
    torch.cuda.synchronize()
    lsa.lsa_timing_reset()
    lsa.lsa_timing_enable(True)
    for _ in range(reps):
        for b in range(nbuf):
            trig(b)
    torch.cuda.synchronize()
    lsa.lsa_timing_enable(False)
    kname = "k_score_sig" if sigmoid else "k_score"
    t = {n: lsa.lsa_timing_read(n) for n in ("k_fuse_query", kname, "k_select")}
    lsa.lsa_timing_reset()
    us = {n: (ms * 1e3 / c if c else None) for n, (c, ms) in t.items()}
    gbs = per / (us[kname] * 1e-6) / 1e9  # per layer launch
    trig_us = sum(ms for (c, ms) in t.values()) * 1e3 / (reps * nbuf)
    del kic, ksc
    torch.cuda.empty_cache()
    out = {"label": label, "batch": B, "context": L,
           "index_keys": "fp8_e4m3fn" if idx_dt == synth.FP8 else "bf16", "indexer_layers": layers,
           "score": "sigmoid" if sigmoid else "relu_fused",
           "bytes_per_trigger": per * layers, "distinct_buffers": nbuf, "launches": reps * nbuf * layers,
           "k_score_us": round(us[kname], 2), "gbs": round(gbs, 1),
           "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
           "trigger_us": round(trig_us, 2)}
    if sigmoid:
        # matrix-core dot products, and (chunk, head) sigmoids on the vector
        # units, per second
        flops = 2.0 * nh * H * d
        out["tflops"] = round(flops / (us[kname] * 1e-6) / 1e12, 1)
        out["sigmoids_per_ns"] = round(nh * H / (us[kname] * 1e3), 1)
    return out


def policy_comparison(inp, n_time=8, mass_steps=64, boost=2.5):
    """The pages' comparison policies on one window of the workload: LSA's
    threshold selection, recency-only (no history chunk), a random 10 % of
    the history chunks, and the top 50 / 25 / 10 % of history chunks by the
    attention mass the full decode of the window's steps gives them.  The
    inputs get an attention focus on the indexer's planted chunks
    (synth.attention_focus) and a cold tier in HBM.  Per policy: chunks
    kept, bytes resident, share of the history's attention mass kept, and
    the time of one decode step (refine, top-k, attention over the kept
    chunks plus the recent window).  Also the attention-mass pass itself."""
    import dataclasses
    import numpy as np
    import torch
    from learned_sparse_kv_amd import lsa, runner, synth
    t0 = time.perf_counter()
    f = synth.attention_focus(inp, boost=boost)
    cfg = dataclasses.replace(inp.cfg, host_cold=False)
    f.cfg = cfg
    dev = runner.DeviceInputs(f)
    B, k = cfg.batch, cfg.topk
    n_hist = [int(x) for x in f["n_hist"]]
    off = [int(x) for x in f["chunk_off"]]
    mass_steps = min(mass_steps, dev.q_attn.shape[0])
    lsa.lsa_timing_reset()
    lsa.lsa_timing_enable(True)
    mass, rec = dev.chunk_mass(dev.q_attn[:mass_steps])
    torch.cuda.synchronize()
    lsa.lsa_timing_enable(False)
    n_ml, ms_ml = lsa.lsa_timing_read("k_chunk_ml")
    lsa.lsa_timing_reset()
    # the pass scores every row of the context against every step's 64 query
    # heads: 2 * Hq * Dk flop per (row, step) on the matrix cores, and it reads
    # each row once per step (the rows of one request fit the caches between
    # steps, so these are not HBM bytes: the distinct bytes are one pass)
    tokens = int(np.sum(f["seq_len"]))
    ml_flops = 2.0 * cfg.Hq * cfg.Dk * tokens * mass_steps
    ml_stream = mass_steps * tokens * cfg.Dk * 2
    ml_unique = tokens * cfg.kv_row_bytes
    ml_tflops = ml_flops / (ms_ml * 1e-3) / 1e12
    share = lambda n, pct: (n * pct + 99) // 100
    pols = {}
    _, sel, cnt = dev.score_select(theta=0.0, window=0)
    pols["lsa"] = (sel, cnt)
    pols["recency_only"] = (torch.zeros_like(sel), torch.zeros_like(cnt))
    pols["random_10pct"] = dev.select_ranked(synth.policy_keys(f), lsa.RANK_SMALLEST_U32,
                                             [share(n, 10) for n in n_hist])
    for pct in (50, 25, 10):
        pols[f"attn_mass_top{pct}pct"] = dev.select_ranked(mass, lsa.RANK_LARGEST_F32,
                                                           [share(n, pct) for n in n_hist])
    hist_mass = float(mass.double().sum())
    rec_total = float(rec.double().sum())
    full_kv = int(np.sum(f["seq_len"])) * cfg.kv_row_bytes
    out = {"workload": cfg.name.replace("hostcold", "hbmcold") + "_window0_attention_focus",
           "attention_focus_boost": boost, "mass_steps": mass_steps,
           "history_mass_share": round(hist_mass / (hist_mass + rec_total), 4),
           "chunk_mass_pass": {"k_chunk_ml_ms": round(ms_ml / max(n_ml, 1), 3), "launches": n_ml,
                               "bound": "mfma", "tflop": round(ml_flops / 1e12, 2),
                               "tflops": round(ml_tflops, 1),
                               "pct_mfma_bf16_peak": round(100 * ml_tflops / MFMA_BF16_PEAK_TFLOPS, 1),
                               "unique_bytes": ml_unique, "unique_gbs": round(ml_unique / (ms_ml * 1e-3) / 1e9, 1),
                               "row_bytes_streamed": ml_stream},
           "policies": {}}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, (sel, cnt) in pols.items():
        torch.cuda.synchronize()
        c = cnt.cpu().numpy()
        keep = torch.zeros_like(mass, dtype=torch.bool)
        s_h = sel.cpu().numpy()
        idx = np.concatenate([off[r] + s_h[off[r]:off[r] + c[r]] for r in range(B)] + [np.zeros(0, np.int64)])
        if len(idx):
            keep[torch.from_numpy(idx.astype(np.int64)).cuda()] = True
        recall = float(mass.double()[keep].sum()) / hist_mass if hist_mass > 0 else 0.0
        for j in range(2):  # warm
            topk, tcnt = dev.refine_topk(sel, cnt, j, k)
            dev.attend(topk, tcnt, j, k)
        torch.cuda.synchronize()
        ev0.record()
        for j in range(n_time):
            topk, tcnt = dev.refine_topk(sel, cnt, j % dev.q_attn.shape[0], k)
            dev.attend(topk, tcnt, j % dev.q_attn.shape[0], k)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / n_time
        kept = int(c.sum())
        resident = kept * cfg.chunk * cfg.kv_row_bytes + int(np.sum(f["n_rec"])) * cfg.kv_row_bytes
        out["policies"][name] = {
            "chunks_kept": kept, "chunk_share": round(kept / max(sum(n_hist), 1), 4),
            "resident_gb": round(resident / 1e9, 3), "resident_share_of_full_kv": round(resident / full_kv, 4),
            "history_mass_recall": round(recall, 4),
            "step_ms": round(ms, 3), "steps_per_s": round(1e3 / ms, 1)}
    del dev, mass, rec, pols
    torch.cuda.empty_cache()
    out["seconds"] = round(time.perf_counter() - t0, 1)
    return out


def window_rate(cfg, n_layers=1, warmup=3, windows=6, steps=64):
    """Decode steps per second of lsa_step64 windows on one workload (inputs
    generated here, cold tier as the config says), with n_layers indexer
    layers selecting their OR union at every trigger.  Wall clock over the
    timed windows, bracketed by device synchronisation."""
    import numpy as np
    import torch
    from learned_sparse_kv_amd import runner, synth
    t0 = time.perf_counter()
    cfg = synth.dataclasses.replace(cfg, windows=warmup + windows + 2, drift=0.02 if cfg.drift == 0 else cfg.drift)
    inp = synth.generate(cfg, steps=steps, threads=16)
    gen_s = time.perf_counter() - t0
    dev = runner.DeviceInputs(inp)
    pipe = runner.Pipeline(dev, n_layers=n_layers)
    B = cfg.batch
    out = torch.empty((steps, B, cfg.Hq, cfg.Dv), dtype=torch.int16, device="cuda")
    _, cnt = pipe.prime()
    m = 0
    for _ in range(warmup):
        pipe.window(m, 0, steps, out)
        m += 1
    torch.cuda.synchronize()
    cnts = []
    t1 = time.perf_counter()
    for _ in range(windows):
        _, c = pipe.window(m, 0, steps, out)
        cnts.append(c)
        m += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    pipe.close()
    res = {"workload": cfg.name, "batch": B, "contexts": [int(x) for x in inp["seq_len"]],
           "index_keys": {0: "f32", 1: "bf16", 2: "fp8_e4m3fn"}[cfg.idx_dtype], "indexer_layers": n_layers,
           "cold_tier": "pinned host" if cfg.host_cold else "HBM", "windows_timed": windows,
           "decode_steps_per_s": round(steps * windows / wall, 1),
           "tokens_per_s": round(B * steps * windows / wall, 1),
           "ms_per_window": round(wall * 1e3 / windows, 3),
           "selected_chunks_per_request": round(float(np.mean(cnts)), 1),
           "generate_s": round(gen_s, 1)}
    del pipe, dev, inp
    torch.cuda.empty_cache()
    return res


def growing_decode(inp, n_windows=7):
    """Growing-context decode through the window pipeline (lsa_step64 with
    a growing context) on the workload's shapes: every request starts
    64 * n_windows tokens short of the workload's context and gains one token
    per step; each window commits the recent region's oldest full chunk,
    which the next trigger (scored one window ahead) already sees.  Cold tier
    as the workload's; the per-step queries repeat after the inputs' 64.
    Window 0 warms up (its commit is the first write to the cold pages),
    window 1 runs with per-kernel timing (append, commit, attention), the
    others are timed by wall clock between device synchronisations."""
    import numpy as np
    import torch
    from learned_sparse_kv_amd import lsa, runner
    cfg = inp.cfg
    B = cfg.batch
    L0 = np.asarray(inp["seq_len"], np.int64) - 64 * n_windows
    t0 = time.perf_counter()
    gp = runner.GrowingPipeline(inp, L0, n_windows, host_cold=cfg.host_cold)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    out = torch.empty((64, B, cfg.Hq, cfg.Dv), dtype=torch.int16, device="cuda")
    gp.prime()
    gp.window(0, out)
    torch.cuda.synchronize()
    lsa.lsa_timing_reset()
    lsa.lsa_timing_enable(True)
    gp.window(1, out)
    torch.cuda.synchronize()
    lsa.lsa_timing_enable(False)
    kt = {}
    for name in ("k_append_kv", "k_commit_page", "k_compact_recent", "k_score", "k_select",
                 "k_refine_mfma", "k_attn_mla"):
        n, ms = lsa.lsa_timing_read(name)
        if n:
            kt[name] = {"launches": n, "avg_us": round(ms * 1e3 / n, 2)}
    lsa.lsa_timing_reset()
    w0 = time.perf_counter()
    for m in range(2, n_windows):
        gp.window(m, out, last=(m == n_windows - 1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    L, rs, _ = gp.state()
    steps = 64 * (n_windows - 2)
    res = {"workload": cfg.name + "_growing", "entry": "lsa_step64 (growing context)",
           "cold_tier": "pinned host" if cfg.host_cold else "HBM",
           "start_context": int(L0[0]), "end_context": int(L[0]), "windows_timed": n_windows - 2,
           "steps_timed": steps, "decode_steps_per_s": round(steps / wall, 1),
           "ms_per_window": round(wall * 1e3 / (n_windows - 2), 3),
           "chunks_committed": int(gp.st["commits"].sum()),
           "history_chunks_end": [int(x) // cfg.chunk for x in rs],
           "kernels_window1": kt, "setup_s": round(setup_s, 1)}
    gp.close()
    del gp
    torch.cuda.empty_cache()
    return res


def sustained_attention(label, B, L, nbatch=6, reps=3, k=2048, Hq=64, Dk=576, Dv=512,
                        window=8192, seed=0):
    """lsa_sparse_decode_attn rotating over nbatch independent batches (pages,
    recent rows, top-k lists, queries), so each launch reads lines no recent
    launch brought into the caches."""
    import numpy as np
    import torch
    from learned_sparse_kv_amd import lsa, synth
    g = lsa.Geom(np.full(B, L, np.int32), window)
    nhist = max(L - window, 0) // 64
    rs = nhist * 64
    nrec = L - rs
    row_bytes, ikey_off = Dk * 2, 64 * Dk * 2
    page_bytes = ikey_off + 64 * 128
    kv = lsa.kv_layout(synth.BF16, Dk, Dv, 0, row_bytes, page_bytes, ikey_off)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    batches = []
    for _ in range(nbatch):
        pages = torch.randn(B * nhist * page_bytes // 2, generator=gen, device="cuda").to(
            torch.bfloat16).view(torch.uint8)
        recent = torch.randn(B * nrec * Dk, generator=gen, device="cuda").to(torch.bfloat16).view(torch.uint8)
        tk = torch.stack([torch.randperm(rs, generator=gen, device="cuda")[:k].sort().values
                          for _ in range(B)]).to(torch.int32).contiguous()
        q = torch.randn(B, Hq, Dk, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
        batches.append((pages, recent, tk, q))
    tcnt = torch.full((B,), k, dtype=torch.int32, device="cuda")
    out = torch.empty(B, Hq, Dv, dtype=torch.int16, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    ws = torch.empty(lsa.lsa_attn_ws_bytes(g, kv, Hq, k, 0), dtype=torch.uint8, device="cuda")

    def run(b):
        pages, recent, tk, q = batches[b]
        lsa.lsa_sparse_decode_attn(g, q, Hq, kv, pages, None, recent, tk, tcnt, k, Dk ** -0.5,
                                   out, lse, 0, ws)

    for b in range(nbatch):
        run(b)
    torch.cuda.synchronize()
    lsa.lsa_timing_reset()
    lsa.lsa_timing_enable(True)
    for _ in range(reps):
        for b in range(nbatch):
            run(b)
    torch.cuda.synchronize()
    lsa.lsa_timing_enable(False)
    c1, ms1 = lsa.lsa_timing_read("k_attn_mla")
    c2, ms2 = lsa.lsa_timing_read("k_attn_merge")
    lsa.lsa_timing_reset()
    toks = B * (k + nrec)
    per = toks * row_bytes + B * Hq * Dk * 2  # rows read + queries
    us = ms1 * 1e3 / c1
    gbs = per / (us * 1e-6) / 1e9
    del batches
    torch.cuda.empty_cache()
    return {"label": label, "batch": B, "context": L, "attended_tokens_per_request": k + nrec,
            "bytes_per_launch": per, "rotating_batches": nbatch, "launches": c1,
            "k_attn_us": round(us, 2), "gbs": round(gbs, 1), "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
            "merge_us": round(ms2 * 1e3 / c2, 2) if c2 else None}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16, help="timed windows (64 decode steps each)")
    ap.add_argument("--warmup", type=int, default=8,
                    help="untimed windows before timing (the first few run slower while the GPU settles)")
    ap.add_argument("--workload", default="cfg4", choices=["cfg1", "cfg2", "cfg3", "cfg4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sustained", action="store_true",
                    help="skip the cold-cache scoring / attention GB/s points at 128K and 500K")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the decode steps/s of the 64K, 128K and 500K batch-4 workloads and of the "
                         "three-layer union")
    ap.add_argument("--no-growing", action="store_true",
                    help="skip the growing-context decode (append per step, chunk commit per window)")
    ap.add_argument("--no-policies", action="store_true",
                    help="skip the comparison policies (recency-only, random 10 %%, attention-mass top shares)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--mfma-calibration", action="store_true",
                    help="also run a bf16 8192^3 GEMM (what matrix-core-bound reads on the counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the LSA decode "
              "path of this library runs every request of a batch on one GPU and has no "
              "multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from learned_sparse_kv_amd import lsa, runner, synth

    torch.cuda.set_device(0)
    # every launch of the run goes to one dedicated stream (the legacy NULL
    # stream would serialise the main work with the refill's copy stream)
    main_stream = torch.cuda.Stream()
    torch.cuda.set_stream(main_stream)
    cfg = synth.config(int(args.workload[3]))
    # one KIComp version per window run (2 % of chunks drift between versions)
    cfg = synth.dataclasses.replace(cfg, windows=args.warmup + args.steps + 3, drift=0.02)
    t0 = time.perf_counter()
    inp = synth.generate(cfg, steps=64, threads=16)
    log(f"[bench] generated {cfg.name} in {time.perf_counter() - t0:.1f}s; "
        f"lens {list(inp['seq_len'][:4])}... history chunks {int(inp['chunk_off'][-1])}")
    dev = runner.DeviceInputs(inp)
    pipe = runner.Pipeline(dev)
    B, S = cfg.batch, 64
    odt = torch.float32 if cfg.kv_dtype == synth.F32 else torch.int16
    out = torch.empty((S, B, cfg.Hq, cfg.Dv), dtype=odt, device="cuda")
    lse = torch.empty((S, B, cfg.Hq), dtype=torch.float32, device="cuda")
    tcnt = torch.empty((S, B), dtype=torch.int32, device="cuda")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st0, cnt = pipe.prime()
    torch.cuda.synchronize()
    prime_s = time.perf_counter() - t0
    log(f"[bench] initial fill: {st0['fetched']} chunks, {st0['bytes'] / 1e6:.1f} MB, {prime_s * 1e3:.1f} ms")

    m = 0
    fetch = []

    def run_window(m, cur_cnt):
        st, nxt_cnt = pipe.window(m, 0, S, out, lse=lse, tcnt=tcnt)
        return st, nxt_cnt

    cur = cnt
    for _ in range(args.warmup):
        st, cur = run_window(m, cur)
        m += 1
    torch.cuda.synchronize()

    # ---- instrumented window (untimed): every kernel bracketed by HIP events
    lsa.lsa_timing_reset()
    lsa.lsa_timing_enable(True)
    win_cnt = cur.copy()
    st, cur = run_window(m, cur)
    m += 1
    torch.cuda.synchronize()
    lsa.lsa_timing_enable(False)
    tsum = int(tcnt.sum().item()) / S  # top-k tokens attended per step (all requests)
    kern = {}
    for name in lsa.KERNELS:
        n, ms = lsa.lsa_timing_read(name)
        if n:
            kern[name] = {"launches": n, "avg_us": round(ms * 1e3 / n, 2), "total_ms": round(ms, 3)}
    lsa.lsa_timing_reset()
    dom = max(kern, key=lambda k_: kern[k_]["total_ms"])
    for name, e in kern.items():
        b, f = kernel_work(name, cfg, inp, win_cnt, cfg.topk, tsum, B)
        sec = e["avg_us"] * 1e-6
        e["alg_bytes"] = int(b)
        e["gbs"] = round(b / sec / 1e9, 1) if b else None
        e["tflops"] = round(f / sec / 1e12, 2) if f else None
    log("[bench] kernels (instrumented window): " + json.dumps(kern))

    # ---- timed region: wall clock for the value; the dominant kernel alone is
    # bracketed by HIP events on its own stream
    lsa.lsa_timing_only(dom)
    lsa.lsa_timing_every(TIMING_EVERY)
    lsa.lsa_timing_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    sel_hist = []
    for _ in range(args.steps):
        sel_hist.append(cur.copy())
        st, cur = run_window(m, cur)
        fetch.append(st)
        m += 1
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lsa.lsa_timing_enable(False)
    dn, dms = lsa.lsa_timing_read(dom)
    lsa.lsa_timing_only(None)
    lsa.lsa_timing_every(1)
    lsa.lsa_timing_reset()
    gpu_ms = ev0.elapsed_time(ev1)
    value = S * args.steps / wall
    log(f"[bench] {args.steps} windows in {wall * 1e3:.1f} ms wall ({gpu_ms:.1f} ms main-stream "
        f"events): {value:.1f} decode steps/s")

    dom_us = dms * 1e3 / dn
    works = [kernel_work(dom, cfg, inp, c, cfg.topk, tsum, B) for c in sel_hist]
    b = sum(x[0] for x in works) / len(works)
    f = sum(x[1] for x in works) / len(works)
    if dom == "k_refine":
        ach = f / (dom_us * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "alu", "achieved": round(ach, 2),
                "peak": round(VALU_F32_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                "frac": round(ach / VALU_F32_PEAK_TFLOPS, 4)}
    else:
        ach = b / (dom_us * 1e-6) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof["avg_us"] = round(dom_us, 2)
    roof["launches_timed"] = dn
    roof["timed_every"] = TIMING_EVERY
    roof["alg_bytes_per_launch"] = int(b)
    roof["traffic"] = traffic_for(dom, cfg.name, dn)

    def hbm(name):
        e = kern.get(name)
        return None if not e or not e.get("gbs") else {"gbs": e["gbs"], "pct_peak": round(100 * e["gbs"] / HBM_PEAK_GBS, 1),
                                                       "avg_us": e["avg_us"]}

    refill_mb = [f["bytes"] / 1e6 for f in fetch]
    ctx = int(inp["seq_len"][0])
    resident = (np.asarray(inp["n_rec"]) + cfg.chunk * win_cnt) / np.asarray(inp["seq_len"])
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "context": ctx,
                   "index_keys": {0: "f32", 1: "bf16", 2: "fp8_e4m3fn"}[cfg.idx_dtype],
                   "topk": cfg.topk, "recent_window": cfg.window,
                   "step": "one lsa_step64 window = 64 decode steps",
                   "cold_tier": "pinned host" if cfg.host_cold else "HBM"},
        "roofline": roof,
        "tokens_per_s": round(value * B, 1),
        "scoring_500k": hbm("k_score"),
        "attention_500k": hbm("k_attn_mla") or hbm("k_attn_f32"),
        "kernels": kern,
        "initial_fill_ms": round(prime_s * 1e3, 2),
        # 256 decode steps from a cold pool: the first trigger and its fill
        # (measured once) plus four windows at the timed rate
        "end_to_end_256_steps": {
            "ms_with_initial_fill": round(prime_s * 1e3 + 4 * wall * 1e3 / args.steps, 2),
            "ms_without_initial_fill": round(4 * wall * 1e3 / args.steps, 2),
            "steps_per_s_with_initial_fill": round(4 * S / (prime_s + 4 * wall / args.steps), 1)},
        "refill_mb_per_window": round(float(np.mean(refill_mb)), 2),
        "selected_chunks_per_request": round(float(win_cnt.mean()), 1),
        "resident_fraction": round(float(resident.mean()), 4),
    }
    if args.copy_calibration:
        a = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()
        del a, bb
    if args.mfma_calibration:
        n = 8192
        a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
        bb = torch.randn((n, n), device="cuda").to(torch.bfloat16)
        cc = torch.mm(a, bb)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            torch.mm(a, bb, out=cc)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / 3
        result["mfma_calibration"] = {"gemm": f"bf16 {n}x{n}x{n}", "avg_us": round(sec * 1e6, 1),
                                      "tflops": round(2 * n ** 3 / sec / 1e12, 1)}
        del a, bb, cc
    pipe.close()
    del pipe, dev
    torch.cuda.empty_cache()
    if not args.no_sustained:
        t0 = time.perf_counter()
        result["hbm_calibration"] = hbm_calibration()
        result["scoring_sustained"] = [
            sustained_scoring("500k", 64, 512000, synth.FP8, seed=101),
            sustained_scoring("128k", 64, 131072, synth.BF16, seed=102),
            sustained_scoring("500k_union3", 64, 512000, synth.FP8, seed=106, layers=3),
            sustained_scoring("500k_sigmoid", 64, 512000, synth.FP8, seed=108, sigmoid=True)]
        result["attention_sustained"] = [
            sustained_attention("500k", 4, 512000, seed=103),
            sustained_attention("500k_b8", 8, 512000, seed=104),
            sustained_attention("128k", 16, 131072, seed=105)]
        ach = result["hbm_calibration"]["stream_read_gbs"]
        for e in result["scoring_sustained"] + result["attention_sustained"]:
            e["pct_achievable_read"] = round(100 * e["gbs"] / ach, 1)
        if roof.get("unit") == "GB/s":
            roof["frac_of_achievable_read"] = round(roof["achieved"] / ach, 4)
        log(f"[bench] sustained points in {time.perf_counter() - t0:.1f}s: "
            + json.dumps({"scoring": result["scoring_sustained"],
                          "attention": result["attention_sustained"]}))
    if not args.no_workloads:
        # decode steps/s at 128K (the ragged 32K-128K batch of 16 and the same
        # batch at 131,072 tokens each) and the pages' three-layer union at 500K
        t0 = time.perf_counter()
        result["decode_steps_128k"] = [window_rate(synth.config(2)), window_rate(synth.config_2u())]
        # the other two window workloads: one request of 64K tokens (bf16 index
        # keys) and 4 requests of 500K (fp8 index keys), both with the HBM cold tier
        result["decode_steps_64k_500k_b4"] = [window_rate(synth.config(1)), window_rate(synth.config(3))]
        # the union of three layers selects about 1 - 0.9^3 = 27 % of the
        # chunks: a pool with room for two windows' selections
        result["union3_window"] = window_rate(synth.dataclasses.replace(cfg, slots_per_req=3072), n_layers=3)
        log(f"[bench] other workloads in {time.perf_counter() - t0:.1f}s: "
            + json.dumps({"128k": result["decode_steps_128k"], "64k_500k_b4": result["decode_steps_64k_500k_b4"],
                          "union3": result["union3_window"]}))
    if not args.no_policies:
        result["policy_comparison"] = policy_comparison(inp)
        log("[bench] policies: " + json.dumps(result["policy_comparison"]))
    if not args.no_growing:
        result["growing_context"] = growing_decode(inp)
        log("[bench] growing context: " + json.dumps(result["growing_context"]))
    if not args.no_cpu_baseline:
        threads = min(16, len(os.sched_getaffinity(0)))
        result["cpu_baseline"] = cpu_baseline(inp, cfg, threads)
        result["cpu_baseline_1core"] = cpu_baseline(inp, cfg, 1, requests=[0])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
