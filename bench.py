#!/usr/bin/env python3
"""Benchmark of the grouped-head attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]
                    [--only WORKLOAD]

One step is one call of the path over one batch of synthetic input, already
resident in HBM.  The headline workload is causal GQA prefill at batch 4,
32 query heads over 8 KV heads, 4096 tokens, head dim 128, bf16 inputs with
fp32 accumulation; `value` is its algorithmic attention TFLOP/s (the causal
pair count times 4*d FLOP, whatever the kernel actually executes).  The other
workloads (the fp32 worked-example shape, GQA decode, GTA shared-score
prefill and decode, latent-absorbed decode, GQLA's per-group paths, paged,
windowed and 8-bit caches) are timed the same way and reported under
"extras".

The CPU leg runs the fp64 oracle (test infrastructure, imported only there)
after each timed GPU workload of the five reference shapes, on the same
seeded inputs: it reports the oracle's own rate ("cpu_baseline") and the
parity of the timed GPU output against it.

Rank 0 prints one JSON line.  Only one GPU is used: --gpus above 1 exits.
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
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from grouped_head_latent_amd import accounting as acc  # noqa: E402

TINY = dict(B=1, h_q=8, h_kv=2, S=16, d=64, seed=0)
PREFILL = dict(B=4, h_q=32, h_kv=8, S=4096, d=128, seed=2)
DECODE = dict(B=64, h_q=32, h_kv=8, d=128, L_lo=1024, L_hi=32768, seed=3)
GTA = dict(B=8, h=16, n_grp=4, S=2048, d=64, seed=4)
LATENT = dict(B=64, h_q=128, r_kv=512, d_r=64, L_lo=8192, L_hi=65536, seed=5, d_h=128)
# decode forms built on the same shapes: GTA's groups at the GQA decode lengths,
# and GQLA's per-group expanded cache (g = 8) at the latent decode lengths
# the decode workload's cache scattered over a shuffled pool of 128-token pages,
# and the same with a 4096-key sliding window
PAGED = dict(page=128, window=4096, seed=8)
GTA_DECODE = dict(B=64, h=16, n_grp=4, d=64, L_lo=1024, L_hi=32768, seed=6)
GQLA_PREFILL = dict(B=2, h_q=128, g=8, S=4096, d_h=128, d_r=64, seed=10, kv_std=0.45)
GQLA_DECODE = dict(B=64, h_q=128, g=8, d_h=128, d_r=64, L_lo=8192, L_hi=65536, seed=7, kv_std=0.45)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel_substr: str):
    """HBM bytes per dispatch of a kernel, from the counter runs recorded in
    profiles/traffic.json (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of
    known size).  None if there is no record or the kernel's source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_substr)
    if rec is None:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec["bytes_per_dispatch"]


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


SPINUP_S = 1.0  # set from --spinup-s
# written before every timed prefill call: larger than the L2s and the MALL
# together, so each call starts with its inputs in HBM only
FLUSH_BYTES = 512 << 20


def time_steps(fn, steps, warmup, torch, flush=None):
    """Spin the GPU clocks up, warm up, then time exactly `steps` calls
    between two synchronisations with HIP events recorded on the stream the
    kernels are launched on.

    With `flush` (a large device buffer) every timed call is preceded by a
    fill of that buffer, which evicts the inputs from L2 and the MALL, and is
    bracketed by its own pair of events; the result is the mean of those
    per-call times (for workloads whose inputs would otherwise stay cached).

    The MI355X ramps its clocks over tens of milliseconds of sustained load;
    a few warmup steps of a sub-millisecond kernel leave it below its steady
    clock.  So the same call first runs untimed for SPINUP_S seconds (not
    counted in `warmup` or `steps`)."""
    # untimed calls follow the same pattern as the timed ones (flush or not),
    # so the clocks settle for that mix of work
    def call(i):
        if flush is not None:
            flush.fill_(i & 127)
        fn()
    t_end = time.perf_counter() + SPINUP_S
    while time.perf_counter() < t_end:
        for i in range(10):
            call(i)
        torch.cuda.synchronize()
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    if flush is not None:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            flush.fill_(i & 127)
            evs[i][0].record(st)
            fn()
            evs[i][1].record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return sum(a.elapsed_time(b) for a, b in evs) / steps, wall
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


# ------------------------------------------------------------------ workloads

def bench_tiny(gha, torch, steps, warmup):
    """The GQA page's worked example shape in fp32: latency of one call."""
    c = TINY
    B, h_q, h_kv, S, d = c["B"], c["h_q"], c["h_kv"], c["S"], c["d"]
    host = [synth.normal_f32(shp, c["seed"], synth.STREAM[n]) for shp, n in
            (((B, h_q, S, d), "q"), ((B, h_kv, S, d), "k"), ((B, h_kv, S, d), "v"))]
    q, k, v = (torch.from_numpy(x).cuda() for x in host)
    o = torch.empty((B, h_q, S, d), dtype=torch.float32, device="cuda")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    ms, wall = time_steps(lambda: gha.gqa_prefill(q, k, v, causal=True, out=o), steps, warmup, torch, flush)
    del flush
    flops = acc.gqa_prefill_flops(B, h_q, S, S, d)
    return dict(us=ms * 1e3, ms=ms, flops=flops, _host=host, _out=o.cpu().numpy())


def bench_prefill(gha, torch, steps, warmup):
    c = PREFILL
    B, h_q, h_kv, S, d = c["B"], c["h_q"], c["h_kv"], c["S"], c["d"]
    q = to_dev(synth.normal_bf16((B, h_q, S, d), c["seed"], 1), torch)
    k = to_dev(synth.normal_bf16((B, h_kv, S, d), c["seed"], 2), torch)
    v = to_dev(synth.normal_bf16((B, h_kv, S, d), c["seed"], 3), torch)
    o = torch.empty((B, h_q, S, d), dtype=torch.bfloat16, device="cuda")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    ms, wall = time_steps(lambda: gha.gqa_prefill(q, k, v, causal=True, out=o), steps, warmup, torch, flush)
    del flush
    flops = acc.gqa_prefill_flops(B, h_q, S, S, d)
    # the output of the last timed call (every call writes the same values)
    return dict(ms=ms, wall=wall, flops=flops, tflops=flops / ms / 1e9,
                bytes=acc.gqa_prefill_bytes(B, h_q, h_kv, S, S, d), _out=o.float().cpu().numpy())


def bench_decode(gha, torch, steps, warmup, s_q):
    c = DECODE
    B, h_q, h_kv, d = c["B"], c["h_q"], c["h_kv"], c["d"]
    L_cap = c["L_hi"]
    seqlens = synth.uniform_i32(B, c["L_lo"], c["L_hi"], c["seed"], synth.STREAM["seqlens"])
    kb = synth.cache_bf16(B, h_kv, L_cap, d, seqlens, c["seed"], 2)
    vb = synth.cache_bf16(B, h_kv, L_cap, d, seqlens, c["seed"], 3)
    qb = synth.normal_bf16((B, h_q, s_q, d), c["seed"], 1)
    kc, vc, q = to_dev(kb, torch), to_dev(vb, torch), to_dev(qb, torch)
    sl = torch.from_numpy(seqlens).cuda()
    o = torch.empty((B, h_q, s_q, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gha.gqa_decode_workspace_bytes(B, h_q, h_kv, s_q, L_cap, d), dtype=torch.uint8, device="cuda")
    ms, wall = time_steps(lambda: gha.gqa_decode(q, kc, vc, sl, out=o, workspace=ws), steps, warmup, torch)
    by = acc.gqa_decode_bytes(seqlens, h_q, h_kv, s_q, d)
    fl = acc.gqa_decode_flops(seqlens, h_q, s_q, d)
    del kc, vc
    return dict(ms=ms, gbps=by / ms / 1e6, tflops=fl / ms / 1e9, bytes=by, flops=fl,
                sum_L=int(seqlens.sum()), _host=(qb, kb, vb, seqlens), _out=o.float().cpu().numpy())


def bench_decode_paged(gha, torch, steps, warmup, s_q, window):
    c, pc = DECODE, PAGED
    B, h_q, h_kv, d = c["B"], c["h_q"], c["h_kv"], c["d"]
    L_cap, page = c["L_hi"], pc["page"]
    seqlens = synth.uniform_i32(B, c["L_lo"], c["L_hi"], c["seed"], synth.STREAM["seqlens"])
    n_pps = L_cap // page
    perm = torch.from_numpy(np.random.default_rng(pc["seed"]).permutation(B * n_pps)).cuda()
    table = torch.empty(B * n_pps, dtype=torch.int32, device="cuda")
    table[perm] = torch.arange(B * n_pps, dtype=torch.int32, device="cuda")
    pools = []
    for stream in (2, 3):
        # page i of sequence b goes to pool page table[b * n_pps + i]
        x = to_dev(synth.cache_bf16(B, h_kv, L_cap, d, seqlens, c["seed"], stream), torch)
        src = x.view(B, h_kv, n_pps, page, d).permute(0, 2, 1, 3, 4).reshape(B * n_pps, h_kv, page, d)
        del x
        pool = torch.empty_like(src)
        pool[table.long()] = src
        del src
        pools.append(pool)
    table = table.view(B, n_pps)
    q = to_dev(synth.normal_bf16((B, h_q, s_q, d), c["seed"], 1), torch)
    sl = torch.from_numpy(seqlens).cuda()
    o = torch.empty((B, h_q, s_q, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gha.gqa_decode_paged_workspace_bytes(B, h_q, h_kv, s_q, L_cap, window, d),
                     dtype=torch.uint8, device="cuda")
    ms, wall = time_steps(lambda: gha.gqa_decode_paged(q, pools[0], pools[1], sl, block_table=table, page_size=page,
                                                       window=window, out=o, workspace=ws), steps, warmup, torch)
    by = acc.gqa_decode_bytes(seqlens, h_q, h_kv, s_q, d, window=window)
    fl = acc.gqa_decode_flops(seqlens, h_q, s_q, d, window=window)
    del pools
    return dict(ms=ms, gbps=by / ms / 1e6, tflops=fl / ms / 1e9, bytes=by, flops=fl,
                keys=acc.windowed_keys(seqlens, s_q, window), page=page, window=window)


def bench_decode_fp8(gha, torch, steps, warmup, s_q):
    """The decode workload with its caches stored as E4M3 codes (scales 1/64)."""
    c = DECODE
    B, h_q, h_kv, d = c["B"], c["h_q"], c["h_kv"], c["d"]
    L_cap = c["L_hi"]
    seqlens = synth.uniform_i32(B, c["L_lo"], c["L_hi"], c["seed"], synth.STREAM["seqlens"])
    ks = vs = 1.0 / 64
    caches = []
    for stream, sc in ((2, ks), (3, vs)):
        x = to_dev(synth.cache_bf16(B, h_kv, L_cap, d, seqlens, c["seed"], stream), torch)
        caches.append((x.float() / sc).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8))
        del x
    q = to_dev(synth.normal_bf16((B, h_q, s_q, d), c["seed"], 1), torch)
    sl = torch.from_numpy(seqlens).cuda()
    o = torch.empty((B, h_q, s_q, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gha.gqa_decode_paged_workspace_bytes(B, h_q, h_kv, s_q, L_cap, 0, d), dtype=torch.uint8,
                     device="cuda")
    ms, wall = time_steps(lambda: gha.gqa_decode_fp8(q, caches[0], caches[1], sl, k_scale=ks, v_scale=vs, out=o,
                                                     workspace=ws), steps, warmup, torch)
    by = acc.gqa_decode_fp8_bytes(seqlens, h_q, h_kv, s_q, d)
    fl = acc.gqa_decode_flops(seqlens, h_q, s_q, d)
    del caches
    return dict(ms=ms, gbps=by / ms / 1e6, tflops=fl / ms / 1e9, bytes=by, flops=fl, sum_L=int(seqlens.sum()))


def bench_gqla_prefill(gha, torch, steps, warmup):
    c = GQLA_PREFILL
    B, h_q, g, S, dh, dr = c["B"], c["h_q"], c["g"], c["S"], c["d_h"], c["d_r"]
    qc = to_dev(synth.normal_bf16((B, h_q, S, dh), c["seed"], 1), torch)
    qr = to_dev(synth.normal_bf16((B, h_q, S, dr), c["seed"], 2), torch)
    kc = to_dev(synth.normal_bf16((B, g, S, dh), c["seed"], 3, c["kv_std"]), torch)
    kr = to_dev(synth.normal_bf16((B, S, dr), c["seed"], 4), torch)
    v = to_dev(synth.normal_bf16((B, g, S, dh), c["seed"], 5, c["kv_std"]), torch)
    o = torch.empty((B, h_q, S, dh), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / float(np.sqrt(dh + dr))
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    ms, wall = time_steps(lambda: gha.gqla_gqa_prefill(qc, qr, kc, kr, v, scale=scale, out=o), steps, warmup,
                          torch, flush)
    del flush
    fl = acc.gqla_prefill_flops(B, h_q, S, S, dh, dr)
    return dict(ms=ms, tflops=fl / ms / 1e9, flops=fl, bytes=acc.gqla_prefill_bytes(B, h_q, g, S, S, dh, dr))


def bench_gta(gha, torch, steps, warmup):
    c = GTA
    B, h, g, S, d = c["B"], c["h"], c["n_grp"], c["S"], c["d"]
    host = (synth.normal_bf16((B, g, S, d), c["seed"], 1), synth.normal_bf16((B, g, S, d), c["seed"], 2),
            synth.normal_bf16((B, h, S, d), c["seed"], 3))
    q, k, v = (to_dev(x, torch) for x in host)
    o = torch.empty((B, h, S, d), dtype=torch.bfloat16, device="cuda")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    ms, wall = time_steps(lambda: gha.gta_shared_score_prefill(q, k, v, out=o), steps, warmup, torch, flush)
    del flush
    fl = acc.gta_prefill_flops(B, h, g, S, d, d)
    return dict(ms=ms, tflops=fl / ms / 1e9, flops=fl, bytes=acc.gta_prefill_bytes(B, h, g, S, d, d),
                _host=host, _out=o.float().cpu().numpy())


def bench_gta_decode(gha, torch, steps, warmup, s_q):
    c = GTA_DECODE
    B, h, g, d = c["B"], c["h"], c["n_grp"], c["d"]
    L_cap = c["L_hi"]
    seqlens = synth.uniform_i32(B, c["L_lo"], c["L_hi"], c["seed"], synth.STREAM["seqlens"])
    kc = to_dev(synth.cache_bf16(B, g, L_cap, d, seqlens, c["seed"], 2), torch)
    vc = to_dev(synth.cache_bf16(B, h, L_cap, d, seqlens, c["seed"], 3), torch)
    q = to_dev(synth.normal_bf16((B, g, s_q, d), c["seed"], 1), torch)
    sl = torch.from_numpy(seqlens).cuda()
    o = torch.empty((B, h, s_q, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gha.gta_shared_score_decode_workspace_bytes(B, h, g, s_q, L_cap, d), dtype=torch.uint8,
                     device="cuda")
    ms, wall = time_steps(lambda: gha.gta_shared_score_decode(q, kc, vc, sl, out=o, workspace=ws), steps, warmup,
                          torch)
    by = acc.gta_decode_bytes(seqlens, h, g, s_q, d, d)
    fl = acc.gta_decode_flops(seqlens, h, g, s_q, d, d)
    del kc, vc
    return dict(ms=ms, gbps=by / ms / 1e6, tflops=fl / ms / 1e9, bytes=by, flops=fl,
                sum_L=int(seqlens.sum()))


def bench_gqla_decode(gha, torch, steps, warmup, s_q):
    c = GQLA_DECODE
    B, h_q, g, d_h, d_r = c["B"], c["h_q"], c["g"], c["d_h"], c["d_r"]
    L_cap = c["L_hi"]
    seqlens = synth.uniform_i32(B, c["L_lo"], c["L_hi"], c["seed"], synth.STREAM["seqlens"])
    kc = to_dev(synth.cache_bf16(B, g, L_cap, d_h, seqlens, c["seed"], synth.STREAM["k"], c["kv_std"]), torch)
    vc = to_dev(synth.cache_bf16(B, g, L_cap, d_h, seqlens, c["seed"], synth.STREAM["v"], c["kv_std"]), torch)
    kr = to_dev(synth.cache_bf16(B, 1, L_cap, d_r, seqlens, c["seed"], synth.STREAM["k_rope"])[:, 0], torch)
    qc = to_dev(synth.normal_bf16((B, h_q, s_q, d_h), c["seed"], synth.STREAM["q_c"]), torch)
    qr = to_dev(synth.normal_bf16((B, h_q, s_q, d_r), c["seed"], synth.STREAM["q_rope"]), torch)
    sl = torch.from_numpy(seqlens).cuda()
    o = torch.empty((B, h_q, s_q, d_h), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gha.gqla_gqa_decode_workspace_bytes(B, h_q, g, s_q, L_cap, d_h), dtype=torch.uint8,
                     device="cuda")
    scale = 1.0 / math.sqrt(d_h + d_r)
    ms, wall = time_steps(lambda: gha.gqla_gqa_decode(qc, qr, kc, kr, vc, sl, scale=scale, out=o, workspace=ws),
                          steps, warmup, torch)
    by = acc.gqla_decode_bytes(seqlens, h_q, g, s_q, d_h, d_r)
    fl = acc.gqla_decode_flops(seqlens, h_q, s_q, d_h, d_r)
    del kc, vc, kr
    return dict(ms=ms, gbps=by / ms / 1e6, tflops=fl / ms / 1e9, bytes=by, flops=fl,
                sum_L=int(seqlens.sum()))


def bench_latent(gha, torch, steps, warmup, s_q):
    c = LATENT
    B, h_q, r, dr = c["B"], c["h_q"], c["r_kv"], c["d_r"]
    L_cap = c["L_hi"]
    seqlens = synth.uniform_i32(B, c["L_lo"], c["L_hi"], c["seed"], synth.STREAM["seqlens"])
    cb = synth.latent_cache_bf16(B, L_cap, r + dr, seqlens, c["seed"], synth.STREAM["latent"])
    qb = synth.normal_bf16((B, s_q, h_q, r), c["seed"], synth.STREAM["q"], 0.25)
    qrb = synth.normal_bf16((B, s_q, h_q, dr), c["seed"], synth.STREAM["q_rope"])
    cache, q_lat, q_r = to_dev(cb, torch), to_dev(qb, torch), to_dev(qrb, torch)
    sl = torch.from_numpy(seqlens).cuda()
    o = torch.empty((B, s_q, h_q, r), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gha.latent_absorb_decode_workspace_bytes(B, h_q, s_q, L_cap, r), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(c["d_h"] + dr)
    ms, wall = time_steps(lambda: gha.latent_absorb_decode(q_lat, q_r, cache[..., :r], cache[..., r:], sl,
                                                           scale=scale, out=o, workspace=ws), steps, warmup, torch)
    by = acc.latent_decode_bytes(seqlens, h_q, s_q, r, dr)
    fl = acc.latent_decode_flops(seqlens, h_q, s_q, r, dr)
    del cache
    return dict(ms=ms, gbps=by / ms / 1e6, tflops=fl / ms / 1e9, bytes=by, flops=fl,
                sum_L=int(seqlens.sum()), _host=(qb, qrb, cb, seqlens, scale), _out=o.float().cpu().numpy())


def bench_absorbing(gha, torch, steps, warmup, s_q):
    """The latent workload with the absorption products on the device:
    content queries q^C and per-group W^UK, W^UV (8 groups, N(0, 0.02^2))."""
    c = LATENT
    B, h_q, r, dr, dh, g = c["B"], c["h_q"], c["r_kv"], c["d_r"], c["d_h"], 8
    L_cap = c["L_hi"]
    seqlens = synth.uniform_i32(B, c["L_lo"], c["L_hi"], c["seed"], synth.STREAM["seqlens"])
    cache = to_dev(synth.latent_cache_bf16(B, L_cap, r + dr, seqlens, c["seed"], synth.STREAM["latent"]), torch)
    q_c = to_dev(synth.normal_bf16((B, s_q, h_q, dh), c["seed"], synth.STREAM["q_c"]), torch)
    q_r = to_dev(synth.normal_bf16((B, s_q, h_q, dr), c["seed"], synth.STREAM["q_rope"]), torch)
    w_uk = to_dev(synth.normal_bf16((g * dh, r), c["seed"], synth.STREAM["w_uk"], 0.02), torch)
    w_uv = to_dev(synth.normal_bf16((g * dh, r), c["seed"], synth.STREAM["w_uv"], 0.02), torch)
    sl = torch.from_numpy(seqlens).cuda()
    o = torch.empty((B, s_q, h_q, dh), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gha.gqla_absorb_decode_workspace_bytes(B, h_q, s_q, L_cap, r), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(dh + dr)
    ms, wall = time_steps(lambda: gha.gqla_absorb_decode(q_c, q_r, w_uk, w_uv, cache[..., :r], cache[..., r:], sl,
                                                         g=g, scale=scale, out=o, workspace=ws), steps, warmup, torch)
    by = acc.absorbing_decode_bytes(seqlens, h_q, g, s_q, dh, r, dr)
    fl = acc.absorbing_decode_flops(seqlens, h_q, s_q, dh, r, dr)
    del cache
    return dict(ms=ms, gbps=by / ms / 1e6, tflops=fl / ms / 1e9, bytes=by, flops=fl, sum_L=int(seqlens.sum()))


# ------------------------------------------------------- CPU leg: the oracle
# The fp64 oracle is test infrastructure; it is imported and run only in the
# functions of this section, on the host, after a workload's GPU timing, on
# the same seeded inputs.  Each leg times the oracle on the full output (or a
# stated bounded sample) and compares the timed GPU output with it.

def _cpu_threads() -> int:
    from threadpoolctl import threadpool_info
    return max([x.get("num_threads", 1) for x in threadpool_info()] + [1])


class Parity:
    """Running max and mean |GPU - oracle| over the compared elements.  For
    bf16 outputs an element also passes when it is within half a bf16 ulp of
    the reference (the output rounding alone reaches 1e-2 at |o| >= 4)."""

    def __init__(self, bf16_out: bool, max_abs: float = 1e-2, mean_abs: float = 1e-3):
        self.bf16_out, self.max_bar, self.mean_bar = bf16_out, max_abs, mean_abs
        self.max, self.sum, self.n, self.over, self.nonfinite = 0.0, 0.0, 0, 0, 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        self.nonfinite += int((~np.isfinite(got)).sum())
        err = np.abs(got - ref)
        allowed = self.max_bar
        if self.bf16_out:
            allowed = np.maximum(self.max_bar, 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7))
        self.over += int((err > allowed).sum())
        self.max = max(self.max, float(np.nanmax(err)) if err.size else 0.0)
        self.sum += float(np.nansum(err))
        self.n += err.size

    def record(self, what: str):
        mean = self.sum / max(self.n, 1)
        ok = self.over == 0 and self.nonfinite == 0 and mean <= self.mean_bar
        return {"max_abs": self.max, "mean_abs": mean, "elements": self.n, "over_bar": self.over,
                "nonfinite": self.nonfinite, "ok": ok, "compared": what,
                "bar": f"max <= {self.max_bar:g}" + (" or half a bf16 ulp" if self.bf16_out else "")
                       + f", mean <= {self.mean_bar:g}"}


def cpu_tiny(res):
    import oracle
    q, k, v = (x.astype(np.float64) for x in res["_host"])
    t0 = time.perf_counter()
    ref, _ = oracle.gqa_prefill(q, k, v, causal=True)
    t = time.perf_counter() - t0
    par = Parity(False, max_abs=1e-5, mean_abs=1e-5)
    par.add(res["_out"], ref)
    return ({"value": t * 1e6, "unit": "us", "cores": _cpu_threads(), "kind": "oracle",
             "sample": "the full output (1 x 8 x 16 x 64, fp32 in, fp64 oracle)"},
            par.record("every element of the timed output"))


def cpu_prefill(res, budget_s=40.0):
    """The oracle on whole (batch, head) slices of the causal prefill, all 128
    unless `budget_s` of oracle time runs out first; the same slices of the
    timed GPU output are compared with it."""
    import oracle
    c = PREFILL
    B, h_q, h_kv, S, d = c["B"], c["h_q"], c["h_kv"], c["S"], c["d"]
    G = h_q // h_kv
    par = Parity(True)
    done, t_total = 0, 0.0
    pairs = [(b, i) for b in range(B) for i in range(h_q)]
    while done < len(pairs) and t_total < budget_s:
        b, i = pairs[done]
        q = oracle.widen_bf16(synth.normal_bf16_rows((B, h_q, S, d), c["seed"], 1, (b, i)))
        k = oracle.widen_bf16(synth.normal_bf16_rows((B, h_kv, S, d), c["seed"], 2, (b, i // G)))
        v = oracle.widen_bf16(synth.normal_bf16_rows((B, h_kv, S, d), c["seed"], 3, (b, i // G)))
        t0 = time.perf_counter()
        ref, _ = oracle.gqa_prefill(q[None, None], k[None, None], v[None, None], causal=True)
        t_total += time.perf_counter() - t0
        par.add(res["_out"][b, i], ref[0, 0])
        done += 1
    flops = done * acc.gqa_prefill_flops(1, 1, S, S, d)
    what = "all" if done == len(pairs) else f"{done} of {len(pairs)}"
    return ({"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": _cpu_threads(), "kind": "oracle",
             "seconds": t_total,
             "sample": f"{what} (batch, head) slices of the causal prefill ({S} x {S} x {d} each), "
                       f"fp64 numpy, {t_total:.1f} s"},
            par.record(f"{what} (batch, head) slices of the timed bf16 output"))


def _decode_rate(by, t, done, total):
    what = "all" if done == total else f"{done} of {total}"
    return {"value": by / t / 1e9, "unit": "GB/s", "cores": _cpu_threads(), "kind": "oracle", "seconds": t,
            "sample": f"{what} sequences ({by / 1e9:.2f} GB of algorithmic traffic), fp64 numpy, {t:.1f} s"}


def cpu_decode(res, s_q, budget_s=60.0):
    import oracle
    c = DECODE
    qb, kb, vb, seqlens = res["_host"]
    par = Parity(True)
    t, done, by = 0.0, 0, 0.0
    for b in range(c["B"]):
        if t >= budget_s:
            break
        L = int(seqlens[b])
        q, k, v = oracle.widen_bf16(qb[b:b + 1]), oracle.widen_bf16(kb[b:b + 1, :, :L]), oracle.widen_bf16(vb[b:b + 1, :, :L])
        t0 = time.perf_counter()
        ref, _ = oracle.gqa_decode(q, k, v, np.array([L]))
        t += time.perf_counter() - t0
        par.add(res["_out"][b:b + 1], ref)
        by += acc.gqa_decode_bytes(seqlens[b:b + 1], c["h_q"], c["h_kv"], s_q, c["d"])
        done += 1
    return _decode_rate(by, t, done, c["B"]), par.record(f"{done} of {c['B']} sequences of the timed bf16 output")


def cpu_gta(res):
    import oracle
    qb, kb, vb = res["_host"]
    q, k, v = (oracle.widen_bf16(x) for x in (qb, kb, vb))
    t0 = time.perf_counter()
    ref, _ = oracle.gta_prefill(q, k, v, causal=True)
    t = time.perf_counter() - t0
    par = Parity(True)
    par.add(res["_out"], ref)
    return ({"value": res["flops"] / t / 1e12, "unit": "TFLOP/s", "cores": _cpu_threads(), "kind": "oracle",
             "seconds": t, "sample": f"the full output, fp64 numpy, {t:.1f} s"},
            par.record("every element of the timed bf16 output"))


def cpu_latent(res, s_q, budget_s=60.0):
    import oracle
    c = LATENT
    qb, qrb, cb, seqlens, scale = res["_host"]
    r = c["r_kv"]
    par = Parity(True)
    t, done, by = 0.0, 0, 0.0
    for b in range(c["B"]):
        if t >= budget_s:
            break
        L = int(seqlens[b])
        cache = oracle.widen_bf16(cb[b:b + 1, :L])
        q, qr = oracle.widen_bf16(qb[b:b + 1]), oracle.widen_bf16(qrb[b:b + 1])
        t0 = time.perf_counter()
        ref, _ = oracle.latent_absorb_decode(q, qr, cache[..., :r], cache[..., r:], np.array([L]), scale=scale)
        t += time.perf_counter() - t0
        par.add(res["_out"][b:b + 1], ref)
        by += acc.latent_decode_bytes(seqlens[b:b + 1], c["h_q"], s_q, r, c["d_r"])
        done += 1
    return _decode_rate(by, t, done, c["B"]), par.record(f"{done} of {c['B']} sequences of the timed bf16 output")


# ------------------------------------------------------------------ provenance

def provenance(torch):
    """CPU model and threads, GPU name and clocks, ROCm and torch versions."""
    import ctypes
    import platform
    env = {"host": platform.node()}
    try:
        with open("/proc/cpuinfo") as f:
            env["cpu_model"] = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        env["cpu_model"] = None
    env["cpu_threads_available"] = len(os.sched_getaffinity(0))
    p = torch.cuda.get_device_properties(0)
    env["gpu_name"] = p.name
    env["gpu_arch"] = getattr(p, "gcnArchName", None)
    env["gpu_cus"] = p.multi_processor_count
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int()
        # hipDeviceAttributeClockRate = 5, hipDeviceAttributeMemoryClockRate = 60
        # (enum hipDeviceAttribute_t in hip_runtime_api.h), both in kHz
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0:
            env["gpu_peak_sclk_mhz"] = val.value / 1000
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 60, 0) == 0:
            env["gpu_peak_mclk_mhz"] = val.value / 1000
    except OSError:
        pass
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        env["rocm"] = None
    env["torch"] = torch.__version__
    env["torch_hip"] = torch.version.hip
    return env


def strip(res):
    """A workload's record without the host arrays the CPU leg used."""
    return {k: v for k, v in res.items() if not k.startswith("_")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle legs (and their parity)")
    ap.add_argument("--only", default=None,
                    help="tiny|prefill|gqla_prefill|decode|paged|paged_window|fp8|gta|latent|absorbing|gta_decode|"
                         "gqla_decode: "
                         "time one workload")
    ap.add_argument("--sq", type=int, default=None, choices=(1, 2),
                    help="decode workloads: time only this many new tokens per sequence")
    ap.add_argument("--spinup-s", type=float, default=1.0,
                    help="untimed seconds of the same workload before the warmup steps (clock ramp)")
    args = ap.parse_args()
    global SPINUP_S
    SPINUP_S = args.spinup_s
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import grouped_head_latent_amd as gha
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gha.load_library()

    only = args.only
    cpu = not args.no_cpu
    extras = {}
    head = None
    head_cpu = head_parity = None

    def run(name, fn, cpu_fn=None):
        log(f"{name} ...")
        res = fn()
        if cpu and cpu_fn is not None:
            log(f"{name}: oracle ...")
            res["cpu_baseline"], res["parity"] = cpu_fn(res)
        res = strip(res)
        log(f"{name}: {res}")
        torch.cuda.empty_cache()
        return res

    want = lambda w: only == w or (only is None and not args.no_extras)
    sqs = (1, 2) if args.sq is None else (args.sq,)
    steps, warmup = args.steps, args.warmup
    if want("tiny"):
        extras["tiny_gqa_fp32"] = run("tiny", lambda: bench_tiny(gha, torch, steps, warmup), cpu_tiny)
    if only in (None, "prefill"):
        log("prefill ...")
        head = bench_prefill(gha, torch, steps, warmup)
        log(f"prefill {head['ms']:.4f} ms {head['tflops']:.1f} TFLOP/s")
        if cpu:
            log("prefill: oracle ...")
            head_cpu, head_parity = cpu_prefill(head)
        head = strip(head)
        torch.cuda.empty_cache()
    if want("gta"):
        extras["gta_prefill"] = run("gta", lambda: bench_gta(gha, torch, steps, warmup), cpu_gta)
    if want("gqla_prefill"):
        extras["gqla_prefill"] = run("gqla prefill", lambda: bench_gqla_prefill(gha, torch, steps, warmup))
    if want("decode"):
        for s_q in sqs:
            extras[f"gqa_decode_sq{s_q}"] = run(f"decode s_q={s_q}",
                                                lambda: bench_decode(gha, torch, steps, warmup, s_q),
                                                lambda r: cpu_decode(r, s_q))
    if want("paged") or only == "paged_window":
        variants = [(s_q, 0) for s_q in sqs] if only != "paged_window" else []
        if only in (None, "paged_window") and 1 in sqs:
            variants.append((1, PAGED["window"]))
        for s_q, window in variants:
            name = f"gqa_decode_paged{PAGED['page']}" + (f"_window{window}" if window else "") + f"_sq{s_q}"
            extras[name] = run(name, lambda: bench_decode_paged(gha, torch, steps, warmup, s_q, window))
    if want("fp8"):
        for s_q in sqs:
            extras[f"gqa_decode_fp8_sq{s_q}"] = run(f"fp8 decode s_q={s_q}",
                                                    lambda: bench_decode_fp8(gha, torch, steps, warmup, s_q))
    if want("latent"):
        for s_q in sqs:
            extras[f"latent_decode_sq{s_q}"] = run(f"latent s_q={s_q}",
                                                   lambda: bench_latent(gha, torch, steps, warmup, s_q),
                                                   lambda r: cpu_latent(r, s_q))
    if want("absorbing"):
        for s_q in sqs:
            extras[f"latent_absorbing_decode_sq{s_q}"] = run(
                f"absorbing latent decode s_q={s_q}", lambda: bench_absorbing(gha, torch, steps, warmup, s_q))
    if want("gta_decode"):
        for s_q in sqs:
            extras[f"gta_decode_sq{s_q}"] = run(f"gta decode s_q={s_q}",
                                                lambda: bench_gta_decode(gha, torch, steps, warmup, s_q))
    if want("gqla_decode"):
        for s_q in sqs:
            extras[f"gqla_decode_sq{s_q}"] = run(f"gqla decode s_q={s_q}",
                                                 lambda: bench_gqla_decode(gha, torch, steps, warmup, s_q))
    for e in extras.values():
        if "gbps" in e:
            e["hbm_frac"] = e["gbps"] / acc.PEAK_HBM_GBPS
        if "tflops" in e:
            e["mfma_frac"] = e["tflops"] / acc.PEAK_BF16_TFLOPS

    env = provenance(torch)
    if head is None:
        print(json.dumps({"extras": extras, "env": env}))
        return
    out = {
        "metric": "decode HBM GB/s (% of peak) + prefill attention TFLOPS (% of MFMA peak)",
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup_s": args.spinup_s,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) rounded to bf16",
        "config": {"workload": "causal GQA prefill, batch 4, 32 query heads / 8 KV heads, "
                               "4096 tokens, head dim 128, bf16 in, fp32 accumulate, bf16 out",
                   "global_batch": PREFILL["B"], "seq_len": PREFILL["S"], "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(head["tflops"], 2), "peak": acc.PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(head["tflops"] / acc.PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("prefill_d128_kernel<2, false, 0>"),
                     "algorithmic_bytes": head["bytes"]},
    }
    if head_cpu is not None:
        out["cpu_baseline"] = head_cpu
        out["parity"] = head_parity
    if extras:
        out["extras"] = extras
    out["env"] = env
    print(json.dumps(out))


if __name__ == "__main__":
    main()
