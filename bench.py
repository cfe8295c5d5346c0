"""Benchmark of the Orthros attention hot path on one MI355X.

One step = one orthros_prefill call on the Llama3.1-8B-shaped 131072-token prompt (32 query /
8 kv heads, d 128, window 4096, bf16, one planted key), i.e. the base stream's windowed rows,
the cache write and the output row at the last token. `value` is prefill tokens/s over the
timed steps, with all inputs already resident in HBM.

The same JSON line carries:
  * roofline: the banded flash kernel (the prefill's dominant kernel): algorithmic FLOPs per
    launch (4 d per (query, key) pair inside the windows, summed over heads) over its mean
    launch time, measured with HIP events the library records around each launch on the
    call's stream during the timed steps; peak = dense bf16 MFMA 2.5 PFLOP/s;
  * decode: the 16 x 131072-token decode workload, 128 consecutive decode steps, as
    microseconds per step and the split-key kernel's algorithmic HBM bytes / launch time
    against 8 TB/s;
  * prefill_chunked: the same prompt fed as 16 chunks of 8192 tokens (orthros_prefill_chunk),
    the output row computed with the last chunk only;
  * sft: the supervised fine-tuning regime at the 1.3B-like shape (batch 4, T 2048, 16 heads,
    window 512) with output rows at the last 512 positions, and its banded kernels' share of
    the bf16 peak;
  * cpu_baseline: the float64 oracle (test infrastructure) timed on this host on a bounded
    sample of the same prefill (base rows at seeded positions, all heads).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-decode] [--skip-cpu]
       [--skip-regimes] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from efficient_attention_amd import orthros as ox  # noqa: E402
from efficient_attention_amd import synthetic as syn  # noqa: E402

PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12      # MI355X HBM3E
CSRC = os.path.join(ROOT, "efficient_attention_amd", "csrc")

# HBM bytes per launch from two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) of
# `bench.py --copy-calibration`, each scaled by what the counter reads for the 1 GiB device copy
# in the same run. Recorded with the sha256 of the kernel's sources (their code: comments and
# blank lines are left out): when the code changes, the figure no longer describes the kernel
# and `traffic` is reported as null.
TRAFFIC = {
    "band_kernel": {"sha": "b2a1f56195090eee", "bytes_per_launch": 2.8647e+09},
    "split_rows_kernel": {"sha": "764e1b6c96dcf5eb", "bytes_per_launch": 8.5959e+09},
    "split_rows_kernel_paged": {"sha": "764e1b6c96dcf5eb", "bytes_per_launch": 8.5969e+09},
}


def kernel_sources_sha(kernel: str) -> str:
    import hashlib
    files = {"band_kernel": ["k_band.hip", "lds_mfma.h"],
             "split_rows_kernel": ["k_split.hip", "lds_mfma.h"],
             "split_rows_kernel_paged": ["k_split.hip", "lds_mfma.h"]}[kernel]
    h = hashlib.sha256()
    for f in files + ["common.h", "launch.h"]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_for(kernel: str):
    rec = TRAFFIC.get(kernel)
    if rec is None or rec["sha"] != kernel_sources_sha(kernel):
        return None
    return rec["bytes_per_launch"]


def copy_calibration(dev, gib=1, reps=3):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {n} bytes (read {n}, write {n} each)")
    del src, dst


def gemm_reference(dev, n=16384, reps=5):
    """A plain bf16 matrix product (torch.matmul, the vendor GEMM library) of n x n x n on the
    same GPU: the dense matrix-core rate this part sustains in practice. Reported beside the
    banded kernel's fraction of the 2.5 PFLOP/s figure, as context; that fraction stays taken
    against the published figure."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / reps
    del a, b, c
    flops = 2.0 * n ** 3
    log(f"gemm reference: {n}^3 bf16 in {s * 1e3:.3f} ms = {flops / s / 1e12:.1f} TFLOP/s")
    return {"kernel": f"torch.matmul bf16 {n}x{n}x{n}", "tflops": round(flops / s / 1e12, 1),
            "frac_of_peak": round(flops / s / PEAK_BF16_FLOPS, 4)}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def swa_pairs(T: int, w: int) -> int:
    """(query, key) pairs inside the windows of Eq. 4 over positions 0..T-1."""
    w = min(w, T)
    return w * (w + 1) // 2 + (T - w) * w


def prefill_flops(wl) -> float:
    d, Hq, B = wl.head_dim, wl.q_heads, wl.batch
    base = 4.0 * d * Hq * B * swa_pairs(wl.length, wl.window)
    out = 4.0 * d * Hq * B * wl.length  # one output row over P keys
    return base, out


def timed(step, steps, reset=None):
    """`steps` calls of step(i) timed with nothing else on the stream (ms per call), then, after
    reset(), the same calls again with the library's per-kernel HIP events on: the stage times
    (the roofline's launch durations) come from that second pass, so the event records never
    sit inside the timed region."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    if reset is not None:
        reset()
        torch.cuda.synchronize()
    ox.timing_begin()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    return ms, ox.timing_end()


def per_step_us(step, steps, reset=None):
    """Each of `steps` calls of step(i) bracketed by HIP events on the current stream (the one
    the library launches on): median and mean microseconds per call. A separate pass, so the
    event records stay out of the timed region."""
    if reset is not None:
        reset()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))
    return us[len(us) // 2], sum(us) / len(us)


def bench_prefill(wl, steps, warmup, dev):
    log(f"prefill {wl.name}: generating inputs on {dev}")
    inp = syn.make_prefill(wl, device=dev)
    B, P, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, P)
    aff = ox.Affine(*inp["affine"])
    ck = torch.empty(B, Hkv, P, d, dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    cl = torch.zeros(B, dtype=torch.int32, device=dev)
    ob = torch.empty(B, P, Hq, d, dtype=torch.bfloat16, device=dev)
    oo = torch.empty(B, 1, Hq, d, dtype=torch.bfloat16, device=dev)
    ws = ox.make_workspace(shape, dev)

    def step():
        ox.prefill(shape, inp["q_base"], inp["q_out"], inp["k"], inp["v"], aff, ck, cv, cl, ob, oo, ws)

    for i in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"prefill warmup {warmup} done; timing {steps} steps")
    ms, stages = timed(lambda i: step(), steps)
    log(f"prefill {ms:.3f} ms/step; stages {stages}")
    return dict(ms=ms, stages=stages, inp=inp, planted=inp["planted_pos"])


def paged_pool(ck, cv, L0, ps, seed):
    """The resident contiguous caches [B, H_kv, cap, d] dealt into a pool of ps-token pages in
    a seeded random order: (k_pages, v_pages, block_table [B, cap / ps] int32)."""
    B, Hkv, cap, d = ck.shape
    assert cap % ps == 0 and L0 % ps == 0
    max_pages, nb = cap // ps, L0 // ps
    g = torch.Generator(device=ck.device)
    g.manual_seed(seed)
    table = torch.randperm(B * max_pages, generator=g, device=ck.device).view(B, max_pages)
    kp = torch.empty(B * max_pages, Hkv, ps, d, dtype=ck.dtype, device=ck.device)
    vp = torch.empty_like(kp)
    for b in range(B):
        kp[table[b, :nb]] = ck[b, :, :L0].reshape(Hkv, nb, ps, d).permute(1, 0, 2, 3)
        vp[table[b, :nb]] = cv[b, :, :L0].reshape(Hkv, nb, ps, d).permute(1, 0, 2, 3)
    return kp, vp, table.to(torch.int32).contiguous()


def bench_decode(wl, warmup, dev, page_size=0):
    """Decode steps over the resident caches; with page_size > 0 over a shuffled page pool."""
    S = wl.steps
    log(f"decode {wl.name}: filling {wl.batch} caches of {wl.length} tokens on {dev}"
        + (f", {page_size}-token pages" if page_size else ""))
    B, L0, Hq, Hkv, d = wl.batch, wl.length, wl.q_heads, wl.kv_heads, wl.head_dim
    cap = L0 + S + warmup
    if page_size:
        cap = -(-cap // page_size) * page_size
    inp = syn.make_decode_resident(wl, dev, cap)
    ck, cv = inp["cache_k"], inp["cache_v"]
    cache = None
    if page_size:
        cache = ox.PagedKV(*paged_pool(ck, cv, L0, page_size, wl.seed + 11))
        # Freed memory stays in torch's allocator here and between the legs: memory returned to
        # the driver (torch.cuda.empty_cache) is cleared by it in the background, and decode
        # steps timed right after returning these 8.6 GB ran 5% slower for ~150 ms.
        inp["cache_k"] = inp["cache_v"] = ck = cv = None
    qb, qo, kn, vn = inp["q_base"], inp["q_out"], inp["k_new"], inp["v_new"]
    aff = ox.Affine(*inp["affine"])
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, cap)
    cl = torch.full((B,), L0, dtype=torch.int32, device=dev)
    ob = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    oo = torch.empty_like(ob)
    ws = ox.make_workspace(shape, dev)

    def step(s, hint):
        if cache is None:
            ox.decode_step(shape, qb[s], qo[s], kn[s], vn[s], aff, ck, cv, cl, hint, ob, oo, ws)
        else:
            ox.decode_step_paged(shape, qb[s], qo[s], kn[s], vn[s], aff, cache, cl, hint, ob, oo,
                                 ws)

    for i in range(warmup):
        step(i % S, L0 + i)
    cl.fill_(L0)
    torch.cuda.synchronize()
    log(f"decode warmup {warmup} done; timing {S} steps")
    ms, stages = timed(lambda s: step(s, L0 + s), S, reset=lambda: cl.fill_(L0))
    assert cl.cpu().tolist() == [L0 + S] * B
    assert ox.read_device_status(ws) == 0
    med, mean_ev = per_step_us(lambda s: step(s, L0 + s), S, reset=lambda: cl.fill_(L0))
    us = ms * 1e3
    # algorithmic bytes: every cached key/value row read once, new k/v read + appended,
    # queries read, outputs written (both streams)
    kv_row = Hkv * d * 2 * 2
    cache_read = sum(B * (L0 + s) * kv_row for s in range(S)) / S
    new_kv = B * kv_row * 2
    qo_bytes = B * Hq * d * 2 * 2 * 2
    step_bytes = cache_read + new_kv + qo_bytes
    split_ms, split_n = stages["split_rows"]
    split_bytes = cache_read + B * kv_row + B * Hq * d * 2 * 2
    split_s = split_ms / 1e3 / max(split_n, 1)
    log(f"decode {us:.1f} us/step; stages {stages}")
    return dict(us=us, stages=stages, step_bytes=step_bytes, split_bytes=split_bytes,
                split_s=split_s, us_median=med, us_mean_events=mean_ev)


def bench_sft(wl, R, steps, warmup, dev):
    """SFT regime: base rows at every position, output rows at the last R positions."""
    inp = syn.make_sft(wl, list(range(wl.length - R, wl.length)), device=dev)
    B, T, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, T)
    aff = ox.Affine(*inp["affine"])
    pos = torch.arange(T - R, T, dtype=torch.int32, device=dev)
    ob = torch.empty(B, T, Hq, d, dtype=torch.bfloat16, device=dev)
    oo = torch.empty(B, R, Hq, d, dtype=torch.bfloat16, device=dev)
    ws = ox.make_workspace(shape, dev, sft_rows=R)

    def step():
        ox.forward_sft(shape, inp["q_base"], inp["q_out"], pos, inp["k"], inp["v"], aff, ob, oo, ws)

    for _ in range(warmup):
        step()
    ms, stages = timed(lambda i: step(), steps)
    flops = 4.0 * d * Hq * B * (swa_pairs(T, wl.window) + sum(t + 1 for t in range(T - R, T)))
    band_ms, band_n = stages["band"]
    log(f"sft {wl.name} R={R}: {ms:.3f} ms/step; stages {stages}")
    return dict(ms=ms, flops=flops, band_ms=band_ms / max(steps, 1))


def bench_training(wl, steps, warmup, dev):
    """Pre-training regime, one training step of the attention: forward with lse + backward."""
    inp = syn.make_pt(wl, device=dev)
    B, T, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, T)
    aff = ox.Affine(*inp["affine"])
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 101)
    do_b = torch.randn(B, T, Hq, d, generator=g, device=dev).to(torch.bfloat16)
    do_o = torch.randn(B, T, Hq, d, generator=g, device=dev).to(torch.bfloat16)
    ob = torch.empty(B, T, Hq, d, dtype=torch.bfloat16, device=dev)
    oo = torch.empty_like(ob)
    lb = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    lo = torch.empty_like(lb)
    ws = ox.make_workspace(shape, dev)
    bws = torch.empty(ox.backward_workspace_bytes(shape, T), dtype=torch.uint8, device=dev)
    dqb, dqo = torch.empty_like(ob), torch.empty_like(ob)
    dk, dv = torch.empty_like(inp["k"]), torch.empty_like(inp["v"])
    dg = [torch.empty(Hq * d, dtype=torch.float32, device=dev) for _ in range(4)]

    def step():
        ox.forward_pt_lse(shape, inp["q_base"], inp["q_out"], inp["k"], inp["v"], aff, ob, oo,
                          lb, lo, ws)
        ox.backward_pt(shape, inp["q_base"], inp["q_out"], inp["k"], inp["v"], aff, ob, oo, lb,
                       lo, do_b, do_o, dqb, dqo, dk, dv, dg, bws)

    for _ in range(warmup):
        step()
    ms, stages = timed(lambda i: step(), steps)
    pairs = B * Hq * (swa_pairs(T, wl.window) + T * (T + 1) // 2)
    fwd_flops = 4.0 * d * pairs
    bwd_flops = 10.0 * d * pairs  # five products per (query, key) pair
    per = {k: v[0] / max(steps, 1) for k, v in stages.items() if v[1]}
    bwd_ms = per.get("bwd_q", 0) + per.get("bwd_kv", 0) + per.get("bwd_affine", 0)
    log(f"training {wl.name}: {ms:.3f} ms/step; stages {per}")
    return dict(ms=ms, per=per, fwd_flops=fwd_flops, bwd_flops=bwd_flops, bwd_ms=bwd_ms,
                pairs=pairs, d=d)


def bench_prefill_chunked(wl, chunk, steps, warmup, dev, inp, page_size=0):
    """The same prompt prefilled in chunks of `chunk` tokens (cache grows chunk by chunk); with
    page_size > 0 into a shuffled pool of pages (cache_len is reset to 0 at the start of each
    step, one small fill kernel). Only the last chunk computes the output-stream row (the
    prompt's last token); the chunks before it pass none."""
    B, P, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    cap = P if not page_size else -(-P // page_size) * page_size
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, cap)
    aff = ox.Affine(*inp["affine"])
    cl = torch.zeros(B, dtype=torch.int32, device=dev)
    if page_size:
        max_pages = cap // page_size
        g = torch.Generator(device=dev)
        g.manual_seed(wl.seed + 13)
        table = torch.randperm(B * max_pages, generator=g, device=dev).view(B, max_pages)
        kp = torch.empty(B * max_pages, Hkv, page_size, d, dtype=torch.bfloat16, device=dev)
        cache = ox.PagedKV(kp, torch.empty_like(kp), table.to(torch.int32).contiguous())
    else:
        ck = torch.empty(B, Hkv, P, d, dtype=torch.bfloat16, device=dev)
        cv = torch.empty_like(ck)
    ws = ox.make_workspace(shape, dev)
    starts = list(range(0, P, chunk))
    views = [(s0, inp["q_base"][:, s0:s0 + chunk].contiguous(), inp["k"][:, s0:s0 + chunk].contiguous(),
              inp["v"][:, s0:s0 + chunk].contiguous()) for s0 in starts]
    obs = [torch.empty(B, q.shape[1], Hq, d, dtype=torch.bfloat16, device=dev) for _, q, _, _ in views]
    oo = torch.empty(B, 1, Hq, d, dtype=torch.bfloat16, device=dev)

    last = starts[-1]

    def step():
        if page_size:
            cl.zero_()
            for (s0, q, k, v), ob in zip(views, obs):
                qo, o = (inp["q_out"], oo) if s0 == last else (None, None)
                ox.prefill_chunk_paged(shape, s0, q, qo, k, v, aff, cache, cl, ob, o, ws)
            return
        for (s0, q, k, v), ob in zip(views, obs):
            qo, o = (inp["q_out"], oo) if s0 == last else (None, None)
            ox.prefill_chunk(shape, s0, q, qo, k, v, aff, ck, cv, cl, ob, o, ws)

    for _ in range(warmup):
        step()
    ms, stages = timed(lambda i: step(), steps)
    log(f"prefill in {len(starts)} chunks of {chunk}" + (f" into {page_size}-token pages" if page_size else "")
        + f": {ms:.3f} ms/step; stages {stages}")
    return dict(ms=ms, chunks=len(starts), band_ms=stages["band"][0] / max(steps, 1))


def host_description():
    """CPUs this process may run on, the machine's CPU count and model, the BLAS thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([x.get("num_threads", 1) for x in threadpool_info()
                    if x.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return dict(usable_cpus=usable, os_cpu_count=os.cpu_count(), cpu_model=model,
                blas_threads=blas)


def cpu_baseline(inp, wl, budget_s=12.0):
    """The float64 oracle on host cores: base rows at seeded positions (all heads)."""
    import oracle
    host = host_description()
    threads = host["blas_threads"]
    log("cpu baseline: copying inputs to host")
    K = inp["k"][0].float().cpu().numpy()
    V = inp["v"][0].float().cpu().numpy()
    a = [x.cpu().numpy() for x in inp["affine"]]
    rng = np.random.default_rng(wl.seed)
    P, w = wl.length, wl.window
    positions = rng.integers(min(w, P - 1), P, size=4000)
    Q = inp["q_base"][0].index_select(0, torch.as_tensor(positions, device=inp["q_base"].device))
    Q = Q.float().cpu().numpy()
    s = oracle.default_scale(wl.head_dim)
    n = 0
    t0 = time.perf_counter()
    while n < len(positions):
        t = int(positions[n])
        oracle.base_row(oracle.scale_offset(Q[n], a[0], a[1]), K, V, t, w, s)
        n += 1
        if time.perf_counter() - t0 > budget_s and n >= 8:
            break
    dt = time.perf_counter() - t0
    log(f"cpu baseline: {n} positions in {dt:.1f} s")
    return dict(value=n / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{n} base-stream positions (all {wl.q_heads} heads, window {w}) drawn "
                       f"uniformly from [{min(w, P - 1)}, {P}) of the {P}-token prompt, "
                       f"float64 numpy, {dt:.1f} s",
                cores_note="cores = the BLAS threads the oracle's products ran on",
                **host)


def all_configs(dev, budget_s=6.0):
    """Each of the five workloads on the GPU next to the float64 oracle on the host cores (a
    bounded sample of each: rows at seeded positions, or whole calls for the tiny one), in the
    workload's own unit. Not part of the default run (`--all-configs`)."""
    import oracle
    out = []
    host = host_description()

    def sample(fn, n_max):
        n, t0 = 0, time.perf_counter()
        while n < n_max:
            fn(n)
            n += 1
            if time.perf_counter() - t0 > budget_s and n >= 2:
                break
        return n, time.perf_counter() - t0

    # tiny fp32 prefill: whole calls
    wl = syn.WORKLOADS["tiny_fp32_prefill"]
    inp = syn.make_prefill(wl)
    B, P, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.float32, P)
    g = {n: inp[n].to(dev) for n in ("q_base", "q_out", "k", "v")}
    aff = ox.Affine(*(a.to(dev) for a in inp["affine"]))
    ck = torch.empty(B, Hkv, P, d, device=dev)
    cv, cl = torch.empty_like(ck), torch.zeros(B, dtype=torch.int32, device=dev)
    ob, oo = torch.empty(B, P, Hq, d, device=dev), torch.empty(B, 1, Hq, d, device=dev)
    ws = ox.make_workspace(shape, dev)
    step = lambda i: ox.prefill(shape, g["q_base"], g["q_out"], g["k"], g["v"], aff, ck, cv, cl,  # noqa: E731
                                ob, oo, ws)
    for _ in range(3):
        step(0)
    ms, _ = timed(step, 50)
    a64 = [a.double().numpy() for a in inp["affine"]]
    h64 = {n: inp[n].double().numpy() for n in ("q_base", "q_out", "k", "v")}
    n, dt = sample(lambda i: oracle.prefill(h64["q_base"], h64["q_out"], h64["k"], h64["v"], *a64,
                                            window=wl.window), 50)
    out.append(dict(workload=wl.name, unit="us per call", gpu=ms * 1e3, oracle=dt / n * 1e6,
                    oracle_sample=f"{n} whole calls"))

    # pre-training forward at the 1.3B shape: both streams at every position
    wl = syn.WORKLOADS["pt_1p3b_2k"]
    inp = syn.make_pt(wl, device=dev)
    B, T, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, T)
    aff = ox.Affine(*inp["affine"])
    ob, oo = (torch.empty(B, T, Hq, d, dtype=torch.bfloat16, device=dev) for _ in range(2))
    ws = ox.make_workspace(shape, dev)
    step = lambda i: ox.forward_pt(shape, inp["q_base"], inp["q_out"], inp["k"], inp["v"], aff,  # noqa: E731
                                   ob, oo, ws)
    for _ in range(3):
        step(0)
    ms, _ = timed(step, 10)
    rng = np.random.default_rng(wl.seed)
    pos = rng.integers(0, T, size=400)
    bs = rng.integers(0, B, size=400)
    K = [inp["k"][b].float().cpu().numpy() for b in range(B)]
    V = [inp["v"][b].float().cpu().numpy() for b in range(B)]
    a64 = [x.cpu().numpy() for x in inp["affine"]]
    qb = inp["q_base"].float().cpu().numpy()
    qo = inp["q_out"].float().cpu().numpy()
    s_ = oracle.default_scale(d)

    def pt_row(i):
        b, t = int(bs[i]), int(pos[i])
        oracle.base_row(oracle.scale_offset(qb[b, t], a64[0], a64[1]), K[b], V[b], t, wl.window, s_)
        oracle.output_row(oracle.scale_offset(qo[b, t], a64[2], a64[3]), K[b], V[b], t, s_)
    n, dt = sample(pt_row, 400)
    out.append(dict(workload=wl.name, unit="tokens/s (both streams)", gpu=B * T / (ms / 1e3),
                    oracle=n / dt, oracle_sample=f"{n} positions at seeded (sequence, position), "
                                                 f"both rows, all {Hq} heads"))
    del inp, ob, oo

    # the two 8B-shaped prefills
    for name in ("prefill_8b_32k", "prefill_8b_128k"):
        wl = syn.WORKLOADS[name]
        pf = bench_prefill(wl, 5, 2, dev)
        cb = cpu_baseline(pf["inp"], wl, budget_s=budget_s)
        out.append(dict(workload=name, unit="tokens/s", gpu=wl.length / (pf["ms"] / 1e3),
                        oracle=cb["value"], oracle_sample=cb["sample"]))
        del pf

    # decode: the GPU step time, and the oracle's decode step for sampled sequences
    dw = syn.WORKLOADS["decode_8b_128k"]
    dc = bench_decode(dw, 4, dev)
    L0, Hq, Hkv, d = dw.length, dw.q_heads, dw.kv_heads, dw.head_dim
    G = Hq // Hkv
    inp = syn.make_decode_resident(dw, dev, L0 + 1)
    a64 = [x.cpu().numpy() for x in inp["affine"]]

    def dec_seq(b):
        for gg in range(Hkv):
            Kg = inp["cache_k"][b, gg, :L0].float().cpu().numpy()[:, None, :]
            Vg = inp["cache_v"][b, gg, :L0].float().cpu().numpy()[:, None, :]
            hs, cs = slice(gg * G, (gg + 1) * G), slice(gg * G * d, (gg + 1) * G * d)
            oracle.decode_step([Kg], [Vg], np.array([L0]),
                               inp["q_base"][0, b:b + 1, hs].float().cpu().numpy(),
                               inp["q_out"][0, b:b + 1, hs].float().cpu().numpy(),
                               inp["k_new"][0, b:b + 1, gg:gg + 1].float().cpu().numpy(),
                               inp["v_new"][0, b:b + 1, gg:gg + 1].float().cpu().numpy(),
                               *(x[cs] for x in a64), window=dw.window)
    n, dt = sample(dec_seq, dw.batch)
    out.append(dict(workload=dw.name, unit="us per step (16 sequences)", gpu=dc["us"],
                    oracle=dt / n * dw.batch * 1e6,
                    oracle_sample=f"{n} of the 16 sequences' first step (L = {L0}), every head, "
                                  f"scaled to 16"))
    return dict(configs=out, host=host)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-regimes", action="store_true",
                    help="skip the SFT and chunked-prefill measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--all-configs", action="store_true",
                    help="only time each of the five workloads on the GPU and the float64 oracle "
                         "on a bounded sample of it, and print that table")
    ap.add_argument("--workload", default="prefill_8b_128k",
                    choices=["prefill_8b_128k", "prefill_8b_32k"])
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    ox.lib()

    if args.all_configs:
        print(json.dumps(all_configs(dev)), flush=True)
        return
    if args.copy_calibration:
        copy_calibration(dev)
    wl = syn.WORKLOADS[args.workload]
    pf = bench_prefill(wl, args.steps, args.warmup, dev)
    base_flops, out_flops = prefill_flops(wl)
    band_ms, band_n = pf["stages"]["band"]
    band_s = band_ms / 1e3 / max(band_n, 1)
    achieved = base_flops / band_s
    tokens = wl.batch * wl.length
    value = tokens / (pf["ms"] / 1e3)
    rec = {
        "metric": "prefill tokens/s @128K (Llama-8B shape)" if wl.length == 131072
        else f"prefill tokens/s @{wl.length // 1024}K (Llama-8B shape)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "prompt_len": wl.length,
                   "q_heads": wl.q_heads, "kv_heads": wl.kv_heads, "head_dim": wl.head_dim,
                   "window": wl.window, "planted_key_pos": pf["planted"],
                   "inputs": "N(0,1) bf16 drawn on cuda:0, seeded"},
        "roofline": {"bound": "mfma", "achieved": round(achieved / 1e12, 2),
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_FLOPS, 4),
                     "traffic": traffic_for("band_kernel"),
                     "kernel": "band_kernel", "launch_ms": round(band_s * 1e3, 4),
                     "flops_per_launch": base_flops},
        "stage_ms_per_step": {k: round(v[0] / max(args.steps, 1), 4)
                              for k, v in pf["stages"].items() if v[1]},
    }
    if not args.skip_decode:
        dw = syn.WORKLOADS["decode_8b_128k"]
        dc = bench_decode(dw, 4, dev)
        ach = dc["split_bytes"] / dc["split_s"]
        rec["decode"] = {
            "metric": "decode-step us @128K", "workload": dw.name, "batch": dw.batch,
            "cache_len": dw.length, "steps": dw.steps, "us_per_step": round(dc["us"], 2),
            "us_per_step_median": round(dc["us_median"], 2),
            "step_GBps": round(dc["step_bytes"] / (dc["us"] / 1e6) / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(ach / 1e9, 1),
                         "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_BYTES, 4),
                         "traffic": traffic_for("split_rows_kernel"),
                         "kernel": "split_rows_kernel", "launch_us": round(dc["split_s"] * 1e6, 2),
                         "bytes_per_launch": dc["split_bytes"]},
            "stage_us_per_step": {k: round(v[0] * 1e3 / dw.steps, 2)
                                  for k, v in dc["stages"].items() if v[1]},
        }
        del dc
        ps = 64
        dp = bench_decode(dw, 4, dev, page_size=ps)
        ach = dp["split_bytes"] / dp["split_s"]
        rec["decode_paged"] = {
            "metric": "decode-step us @128K", "workload": f"{dw.name}, paged",
            "page_size": ps, "pages": "shuffled pool, one block table row per sequence",
            "us_per_step": round(dp["us"], 2), "us_per_step_median": round(dp["us_median"], 2),
            "roofline": {"bound": "hbm", "achieved": round(ach / 1e9, 1),
                         "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_BYTES, 4),
                         "traffic": traffic_for("split_rows_kernel_paged"),
                         "kernel": "split_rows_kernel (paged)",
                         "launch_us": round(dp["split_s"] * 1e6, 2),
                         "bytes_per_launch": dp["split_bytes"]},
            "stage_us_per_step": {k: round(v[0] * 1e3 / dw.steps, 2)
                                  for k, v in dp["stages"].items() if v[1]},
        }
    if not args.skip_regimes:
        ch = bench_prefill_chunked(wl, 8192, max(2, args.steps // 3), 1, dev, pf["inp"])
        rec["prefill_chunked"] = {
            "workload": f"{wl.name} in chunks of 8192, output row with the last chunk",
            "chunks": ch["chunks"],
            "ms_per_step": round(ch["ms"], 4), "tokens_per_s": round(tokens / (ch["ms"] / 1e3), 1),
            "band_frac": round(base_flops / (ch["band_ms"] / 1e3) / PEAK_BF16_FLOPS, 4),
        }
        chp = bench_prefill_chunked(wl, 8192, max(2, args.steps // 3), 1, dev, pf["inp"],
                                    page_size=64)
        rec["prefill_chunked_paged"] = {
            "workload": f"{wl.name} in chunks of 8192 into a shuffled pool of 64-token pages, "
                        "output row with the last chunk",
            "chunks": chp["chunks"], "ms_per_step": round(chp["ms"], 4),
            "tokens_per_s": round(tokens / (chp["ms"] / 1e3), 1),
            "band_frac": round(base_flops / (chp["band_ms"] / 1e3) / PEAK_BF16_FLOPS, 4),
        }
        sw = syn.WORKLOADS["pt_1p3b_2k"]
        sf = bench_sft(sw, 512, args.steps, args.warmup, dev)
        rec["sft"] = {
            "workload": f"{sw.name}, response rows at the last 512 positions",
            "ms_per_step": round(sf["ms"], 4),
            "tokens_per_s": round(sw.batch * sw.length / (sf["ms"] / 1e3), 1),
            "roofline": {"bound": "mfma", "achieved": round(sf["flops"] / (sf["band_ms"] / 1e3) / 1e12, 2),
                         "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                         "frac": round(sf["flops"] / (sf["band_ms"] / 1e3) / PEAK_BF16_FLOPS, 4),
                         "kernel": "band_kernel (both row sets, one launch)"},
        }
    if not args.skip_regimes:
        tw = syn.WORKLOADS["pt_1p3b_2k"]
        tr = bench_training(tw, args.steps, args.warmup, dev)
        per = tr["per"]
        ach = tr["bwd_flops"] / (tr["bwd_ms"] / 1e3)
        rec["training"] = {
            "workload": f"{tw.name}: forward with log-sum-exp + backward, both streams",
            "ms_per_step": round(tr["ms"], 4),
            "tokens_per_s": round(tw.batch * tw.length / (tr["ms"] / 1e3), 1),
            "forward_ms": round(per.get("band", 0), 4), "backward_ms": round(tr["bwd_ms"], 4),
            "stage_ms_per_step": {k: round(v, 4) for k, v in per.items()},
            "roofline": {"bound": "mfma", "achieved": round(ach / 1e12, 2),
                         "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                         "frac": round(ach / PEAK_BF16_FLOPS, 4),
                         "kernel": "backward (bwd_q + bwd_kv + scale-offset), 10 d FLOP per pair",
                         "flops_per_step": tr["bwd_flops"]},
            "kernel_tflops": {
                "bwd_q": round(6.0 * tr["d"] * tr["pairs"] / (per.get("bwd_q", 1) / 1e3) / 1e12, 1),
                "bwd_kv": round(8.0 * tr["d"] * tr["pairs"] / (per.get("bwd_kv", 1) / 1e3) / 1e12, 1)},
            "gradient_tolerance": "per gradient tensor, against the float64 oracle: mean relative "
                                  "error <= 5e-3 and max-abs <= 1e-2 x the tensor's largest "
                                  "magnitude; a bf16 gradient passes through up to four bf16 "
                                  "roundings (post-affine query, probabilities, score gradient, "
                                  "the forward output inside D), each <= 2^-9 relative",
        }
    # last of the GPU legs: the product draws the most power of anything here, and a leg timed
    # right after it (the decode step) read ~5% slower
    ref = gemm_reference(dev)
    ref["band_vs_gemm"] = round(achieved / 1e12 / ref["tflops"], 4)
    rec["roofline"]["gemm_reference"] = ref
    if not args.skip_cpu:
        rec["cpu_baseline"] = cpu_baseline(pf["inp"], wl)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
