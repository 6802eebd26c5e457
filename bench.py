#!/usr/bin/env python3
"""Benchmark of partitioned attention over a ring-buffer KV cache on one MI355X.

Headline workload (the default): the long-history configuration, 18 layers,
8 query heads sharing 1 KV head of width 256, bf16; a pinned prefix of 256
tokens and a sliding window of 8 frames x 768 tokens in the ring; a 51-token
dynamic suffix; 10 denoising steps per frame. One headline step is one
partitioned-attention pass over all 18 layers at once (layer-batched: every
layer's suffix Q/K/V of the step is given; split-KV partials + log-sum-exp
combine). Each ring pushes a new frame (evicting the oldest) before every
10th of its own steps, and the rings' frame boundaries are staggered so that
pushes fall inside any timed window of 10 or more steps; the push count in
the timed region is reported. Inputs are seeded synthetic tensors already
resident in HBM. The headline is the cold case: three independent rings
(sessions) are served round-robin, so each step's 118 MB of K/V comes from
HBM rather than the 256 MB last-level cache; the single-ring (warm) figure
is reported beside it, as are microseconds per call on the two small
configurations.

Each workload first runs its own loop untimed for --settle-ms (250 ms by
default) before its warmup steps: the matrix-core kernels run 15-25% slower
for their first few hundred launches after the GPU has idled, so without it
a short timed region measures that transient rather than the steady state of
a running loop. The headline reports the mean of its first 100 launches
(config.settle) beside the settled figures.

Reported beside it in the same JSON line:
* the chained denoising step on the long-history cache (norm -> packed QKV ->
  attention -> out-projection with residual, layer by layer, 18 layers,
  Euler update), replayed as a captured graph, in microseconds per step:
  this is the step a real loop runs, since layer l + 1's Q needs layer l's
  output;
* the same chained step of the Pi0.5-like 18-layer stack (48 + 2 x 768
  token cache), with and without the SwiGLU FFN;
* the shared-KV multi-reader frame (the action suffix plus 16 decode streams
  with private tails over the long-history cache), in frames/s and decode
  tokens/s.

``roofline`` describes the split-KV partial kernel of the headline step,
timed in a separate pass of at least 20 launches with HIP events recorded
around it on the launch stream (same cold round-robin). ``cpu_baseline`` is
the float64 CPU oracle timed on bounded samples of the long-history step,
the Pi0.5-like single-layer step and the Pi0.5-like 18-layer stack step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "denoise steps/sec + HBM GB/s (% roofline), Pi0.5-like 18L partitioned attn"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def settle(torch, ms, step, chunk):
    """Run the workload's own loop, step(i) for i = 0, 1, ..., untimed, for
    `ms` milliseconds of wall time; return the number of calls made.

    On this GPU the matrix-core kernels run 15-25% slower for their first few
    hundred launches after the device has been idle for as little as 0.2 s,
    while the shader clock and HBM copy bandwidth hold steady; the slowdown
    fades over about 40 ms of continuous work whatever the K/V footprint (the
    same with 118 MB and 708 MB of rings). A serving loop runs continuously,
    so the settle phase runs before the warmup steps and the timed steps
    measure the steady state. The host keeps one chunk of calls queued
    behind the running one, so the GPU does not idle in between."""
    if ms <= 0:
        return 0
    i, pending = 0, None
    t_end = time.perf_counter() + ms / 1e3
    while True:
        for _ in range(chunk):
            step(i)
            i += 1
        ev = torch.cuda.Event()
        ev.record()
        if pending is not None:
            pending.synchronize()
        pending = ev
        if time.perf_counter() >= t_end:
            break
    torch.cuda.synchronize()
    return i


class KernelEvents:
    """HIP timing events created without the system-scope fence
    (hipEventDisableSystemFence), from the HIP runtime torch has loaded.
    A default timing event writes back and invalidates the caches when it is
    recorded: around the partial kernel that adds the write-back of its
    27 MB of partials and a cold start to the measurement. These events time
    the launch as it runs between unmarked steps."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes as C
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.C, self.hip = C, C.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.made = []

    def pair(self):
        evs = []
        for _ in range(2):
            ev = self.C.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(self.C.byref(ev), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            evs.append(ev.value)
            self.made.append(ev.value)
        return tuple(evs)

    def elapsed_ms(self, a, b) -> float:
        ms = self.C.c_float()
        rc = self.hip.hipEventElapsedTime(self.C.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ev)
        self.made = []


def attention_work(s, cached_tokens):
    """Algorithmic bytes and flops of one partial-kernel launch over all layers.

    Bytes: the cached K and V read once, plus Q and the suffix K/V (partials,
    padding and the combine's output are not counted). Flops: QK^T and PV,
    2 * M * T * D each, M = tokens x heads, T = cached + suffix keys.
    """
    L, D, hq, hkv, n = s.num_layers, s.head_dim, s.n_q_heads, s.n_kv_heads, s.n_dyn
    kv_cached = 2 * L * cached_tokens * hkv * D * 2
    q_bytes = L * n * hq * D * 2
    dyn = 2 * L * n * hkv * D * 2
    t = cached_tokens + n
    flops = 2 * 2 * L * n * hq * t * D
    return kv_cached + q_bytes + dyn, flops, kv_cached


def bench_long_history(args, torch, L, configs, synth, n_rings=1, q_layout=0, partials_f32=0):
    """The headline step. With n_rings > 1, that many independent rings (one
    per session) are served round-robin, one step each in turn; three rings
    hold 354 MB of K/V, more than the 256 MB last-level cache (MALL), so
    every step streams its ring's K/V from HBM (the cold case). One ring of
    118 MB stays resident in the MALL between steps (the warm case)."""
    s = configs.LONG_18L
    dev = lambda a: torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda()  # noqa: E731
    shp = (s.num_layers, s.max_seq_len, s.n_kv_heads, s.head_dim)
    pk, pv = synth.pin_kv(s)
    log("generating the frame pool and step inputs")
    pool = [tuple(dev(a) for a in synth.frame_kv(s, f)) for f in range(4)]
    steps_in = [tuple(dev(a) for a in synth.suffix_qkv(s, 0, k)) for k in range(s.steps_per_frame)]
    rings, bufs = [], []
    for r in range(n_rings):
        k_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
        v_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
        ring = L.Ring(L.rb_config(s.num_layers, s.n_kv_heads, s.head_dim, s.pin_tokens, s.num_slots,
                                  s.tokens_per_frame, L.PA_BF16), k_buf, v_buf)
        ring.pin_prefix(dev(pk), dev(pv), s.pin_tokens)
        for f in range(s.num_slots):
            ring.push_frame(*pool[(f + r) % 4])
        rings.append(ring)
        bufs.append((k_buf, v_buf))
    args_ = L.pattn_args(0, s.num_layers, s.n_q_heads, s.n_dyn, s.scale, L.PA_BF16, args.splits, q_layout,
                         partials_f32)
    if q_layout == L.PA_Q_OPERAND:
        # Q in the kernel's operand order, as a producer that writes Q (the
        # stack's QKV projection) lays it out; converted once, before timing
        def operand(q):
            qo = torch.empty(L.pattn_operand_q_bytes(rings[0], args_) // 2, dtype=torch.int16, device="cuda")
            L.pattn_pack_q(rings[0], args_, q, qo)
            return qo
        steps_in = [(operand(q), kd, vd) for q, kd, vd in steps_in]
    wsb = L.pattn_workspace_bytes(rings[0], args_)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((s.num_layers, s.n_dyn, s.n_q_heads, s.head_dim), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    frame = [s.num_slots] * n_rings
    spf = s.steps_per_frame
    # Ring r serves global steps i = j * n_rings + r (its own step j) and
    # pushes before its own steps j with (j + phase_r) % spf == 0; the phases
    # spread the rings' frame boundaries evenly, so globally a push falls
    # about every spf steps and any timed window of spf or more steps holds one.
    phase = [(r * spf) // n_rings for r in range(n_rings)]
    pushes = [0]

    def one_step(i, ev=None):
        r, j = i % n_rings, i // n_rings         # ring, and that ring's own step count
        if (j + phase[r]) % spf == 0:
            rings[r].push_frame(*pool[frame[r] % 4])
            frame[r] += 1
            pushes[0] += 1
        q, kd, vd = steps_in[(j + phase[r]) % spf]
        if ev is None:
            L.pattn_step(rings[r], args_, q, kd, vd, out, ws, wsb, stream)
        else:
            L.pattn_step_timed(rings[r], args_, q, kd, vd, out, ws, wsb, stream, ev[0], ev[1])

    # The first launches of the loop, each timed (enqueued behind a spin
    # kernel, as the roofline pass below is): the unsettled figure. One
    # untimed step goes first, so that the runtime's one-time loading of the
    # kernels' code objects on their first launch is not in it.
    n_first = 100 if args.settle_ms > 0 else 0
    kev = KernelEvents()
    evs = [kev.pair() for _ in range(n_first)]
    if n_first:
        one_step(0)
        torch.cuda.synchronize()
        torch.cuda._sleep(4_000_000)
    for i in range(n_first):
        one_step(1 + i, evs[i])
    n_first += 1 if n_first else 0
    n_settle = n_first + settle(torch, args.settle_ms, lambda i: one_step(n_first + i), 50)
    for i in range(args.warmup):
        one_step(n_settle + i)
    torch.cuda.synchronize()
    first_ms = [kev.elapsed_ms(a, b) for a, b in evs]
    pushes[0] = 0
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(n_settle + args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    pushes_timed = pushes[0]
    # Roofline pass: the partial kernel timed alone on every launch of a
    # further stretch of the same loop (an event pair around every launch
    # adds dispatch latency, so this pass is kept out of the throughput).
    n_kern = max(args.kernel_launches, 20)
    evs = [kev.pair() for _ in range(n_kern)]
    base = n_settle + args.warmup + args.steps
    # The pass is enqueued behind a short spin kernel (about 2 ms), so that
    # the host is far enough ahead that no launch waits for its enqueue: with
    # the queue empty, an event pair measured a launch plus the gap to the
    # host's next submission (71-72 us after a 20-step run, against 59-62 us
    # after a 600-step run on the same box).
    torch.cuda._sleep(4_000_000)
    for i in range(n_kern):
        one_step(base + i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [kev.elapsed_ms(a, b) for a, b in evs]
    kev.close()
    if not kern_ms:
        raise RuntimeError("no partial-kernel launch was timed")
    avg_kern_s = sum(kern_ms) / len(kern_ms) / 1e3
    sd = (sum((k / 1e3 - avg_kern_s) ** 2 for k in kern_ms) / len(kern_ms)) ** 0.5
    # one push alone (both tensors of all 18 layers), averaged over a few
    push_ev0, push_ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_push = 8
    push_ev0.record()
    for i in range(n_push):
        rings[i % n_rings].push_frame(*pool[i % 4])
    push_ev1.record()
    torch.cuda.synchronize()
    t_push = push_ev0.elapsed_time(push_ev1) / n_push / 1e3
    cached = s.pin_tokens + s.num_slots * s.tokens_per_frame
    algo_bytes, flops, kv_bytes = attention_work(s, cached)
    t_step = elapsed / args.steps
    res = {
        "elapsed_s": elapsed,
        "steps_per_s": args.steps / elapsed,
        "ms_per_step": t_step * 1e3,
        "pushes_timed": pushes_timed,
        "push_us": t_push * 1e6,
        "partial_us": avg_kern_s * 1e6,
        "partial_us_sd": sd * 1e6,
        "partial_us_min": min(kern_ms) * 1e3,
        "partial_us_max": max(kern_ms) * 1e3,
        "timed_launches": len(kern_ms),
        "partial_tflops": flops / avg_kern_s / 1e12,
        "partial_gbs": algo_bytes / avg_kern_s / 1e9,
        "kv_gbs_step": kv_bytes / t_step / 1e9,
        "algo_bytes": algo_bytes,
        "flops": flops,
        "splits": args.splits,
        "rings": n_rings,
        "q_layout": "operand" if q_layout else "token_major",
        "partials": "fp32" if partials_f32 else "bf16",
        "settle_steps": n_settle,
        "first_launches_us": sum(first_ms) / len(first_ms) * 1e3 if first_ms else None,
    }
    for ring in rings:
        ring.close()
    return res


def bench_async_push(args, torch, L, configs, synth, n_frames=40):
    """Frames/s of the long-history workload on a ring with a spare slot:
    pushes on the denoising stream (synchronous) against frames staged on a
    producer stream while the previous frame's ten steps run (overlapped)."""
    s = configs.LONG_18L
    dev = lambda a: torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda()  # noqa: E731
    seq = s.pin_tokens + (s.num_slots + 1) * s.tokens_per_frame
    shp = (s.num_layers, seq, s.n_kv_heads, s.head_dim)
    k_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
    v_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
    ring = L.Ring(L.rb_config(s.num_layers, s.n_kv_heads, s.head_dim, s.pin_tokens, s.num_slots,
                              s.tokens_per_frame, L.PA_BF16, 1), k_buf, v_buf)
    pk, pv = synth.pin_kv(s)
    ring.pin_prefix(dev(pk), dev(pv), s.pin_tokens)
    pool = [tuple(dev(a) for a in synth.frame_kv(s, f)) for f in range(4)]
    steps_in = [tuple(dev(a) for a in synth.suffix_qkv(s, 0, k)) for k in range(s.steps_per_frame)]
    for f in range(s.num_slots + 1):
        ring.push_frame(*pool[f % 4])
    args_ = L.pattn_args(0, s.num_layers, s.n_q_heads, s.n_dyn, s.scale, L.PA_BF16, args.splits)
    wsb = L.pattn_workspace_bytes(ring, args_)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((s.num_layers, s.n_dyn, s.n_q_heads, s.head_dim), dtype=torch.int16, device="cuda")
    consumer, producer = torch.cuda.current_stream(), torch.cuda.Stream()

    def steps():
        for k in range(s.steps_per_frame):
            q, kd, vd = steps_in[k]
            L.pattn_step(ring, args_, q, kd, vd, out, ws, wsb, consumer)

    def run_sync(n):
        for f in range(n):
            ring.push_frame(*pool[f % 4], consumer)
            steps()

    def run_async(n):
        for f in range(n):
            ring.commit_frame(consumer)               # frame f joins the window
            ring.stage_frame(*pool[(f + 1) % 4], producer)   # frame f+1 fills the spare meanwhile
            steps()

    res = {}
    for name, fn in (("sync", run_sync), ("async", None)):
        if name == "async":
            ring.stage_frame(*pool[0], producer)
            fn = run_async
        fn(3)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn(n_frames)
        torch.cuda.synchronize()
        res[name] = n_frames / (time.perf_counter() - t0)
    ring.commit_frame(consumer)
    torch.cuda.synchronize()
    ring.close()
    return {"workload": "long_history_18L, window of 8 frames plus one spare slot",
            "frames_per_s_sync_push": res["sync"], "frames_per_s_overlapped_push": res["async"],
            "us_per_frame_sync": 1e6 / res["sync"], "us_per_frame_overlapped": 1e6 / res["async"],
            "frames_timed": n_frames}


def bench_small(args, torch, L, cfg, n_calls=2000):
    """Microseconds per pattn_step call on a small, launch-latency-bound
    configuration (whole window full)."""
    dt = torch.float32 if cfg.dtype == "f32" else torch.int16
    pdt = L.PA_F32 if cfg.dtype == "f32" else L.PA_BF16
    from partitioned_kv_cache_amd import synth
    dev = lambda a: torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda()  # noqa: E731
    shp = (cfg.num_layers, cfg.max_seq_len, cfg.n_kv_heads, cfg.head_dim)
    k_buf, v_buf = torch.zeros(shp, dtype=dt, device="cuda"), torch.zeros(shp, dtype=dt, device="cuda")
    ring = L.Ring(L.rb_config(cfg.num_layers, cfg.n_kv_heads, cfg.head_dim, cfg.pin_tokens, cfg.num_slots,
                              cfg.tokens_per_frame, pdt), k_buf, v_buf)
    pk, pv = synth.pin_kv(cfg)
    ring.pin_prefix(dev(pk), dev(pv), cfg.pin_tokens)
    for f in range(cfg.num_slots):
        ring.push_frame(*(dev(a) for a in synth.frame_kv(cfg, f)))
    q, kd, vd = (dev(a) for a in synth.suffix_qkv(cfg, 0, 0))
    a = L.pattn_args(0, cfg.num_layers, cfg.n_q_heads, cfg.n_dyn, cfg.scale, pdt, 0)
    wsb = L.pattn_workspace_bytes(ring, a)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.num_layers, cfg.n_dyn, cfg.n_q_heads, cfg.head_dim), dtype=dt, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(50):
        L.pattn_step(ring, a, q, kd, vd, out, ws, wsb, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_calls):
        L.pattn_step(ring, a, q, kd, vd, out, ws, wsb, stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # the same calls captured in a graph (no host launch cost), timed with events
    per_graph = 20
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        cs = torch.cuda.current_stream()
        for _ in range(per_graph):
            L.pattn_step(ring, a, q, kd, vd, out, ws, wsb, cs)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(1, n_calls // per_graph)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    g_us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
    ring.close()
    return {"workload": cfg.name, "us_per_call": el / n_calls * 1e6, "us_per_call_graph": g_us, "calls": n_calls,
            "cached_tokens": cfg.max_seq_len, "suffix": cfg.n_dyn, "layers": cfg.num_layers}


def bench_adanorm_qkv(args, torch, L, configs, synth, n_calls=2000):
    """One layer's fused AdaRMSNorm + packed QKV projection (ada_rmsnorm_qkv)
    at the Pi0.5-like shape: 51 rows of a 1024-wide stream, W_qkv 1024 ->
    (8 + 2) x 256. Microseconds per call, eager and graph-replayed, and the
    rate over the bytes the call must move (weights, x, gamma, q/k/v)."""
    s = configs.PI05_18L
    dev = lambda a: torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda()  # noqa: E731
    rows, model, hq, hkv, d = s.n_dyn, s.model_dim, s.n_q_heads, s.n_kv_heads, s.head_dim
    x = dev(synth.normal((rows, model), "bf16", s.cfg_id, synth.T_X, 9))
    w = dev(synth.proj_weights(s, 0)[0])
    gam = torch.ones(model, dtype=torch.float32, device="cuda")
    q = torch.empty((rows, hq, d), dtype=torch.int16, device="cuda")
    k = torch.empty((rows, hkv, d), dtype=torch.int16, device="cuda")
    v = torch.empty((rows, hkv, d), dtype=torch.int16, device="cuda")
    wsb = L.ada_rmsnorm_qkv_workspace_bytes(rows, model)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call(st):
        L.ada_rmsnorm_qkv(x, rows, model, gam, s.eps, w, hq, hkv, d, q, k, v, None, ws, wsb, st)

    for _ in range(50):
        call(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_calls):
        call(stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    per_graph = 20
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        cs = torch.cuda.current_stream()
        for _ in range(per_graph):
            call(cs)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(1, n_calls // per_graph)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    g_us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
    n_out = (hq + 2 * hkv) * d
    algo = model * n_out * 2 + rows * model * 2 + model * 4 + rows * n_out * 2
    return {"workload": "pi05_like_adarmsnorm_qkv_1L", "rows": rows, "model_dim": model, "qkv_dim": n_out,
            "us_per_call": round(el / n_calls * 1e6, 2), "us_per_call_graph": round(g_us, 2),
            "algo_bytes": algo, "gbs_graph": round(algo / (g_us * 1e-6) / 1e9, 1)}


def bench_capsule(args, torch, L, configs, synth, n_calls=50):
    """Row f4: rb_snapshot / rb_restore of the long-history ring (18 layers,
    pin 256 + 8 x 768 tokens, window wrapped so each copy is split into its
    physical runs) into a device capsule; microseconds per call and the copy
    rate over 2 x capsule bytes (read and write)."""
    s = configs.LONG_18L
    dev = lambda a: torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda()  # noqa: E731
    shp = (s.num_layers, s.max_seq_len, s.n_kv_heads, s.head_dim)
    k_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
    v_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
    ring = L.Ring(L.rb_config(s.num_layers, s.n_kv_heads, s.head_dim, s.pin_tokens, s.num_slots,
                              s.tokens_per_frame, L.PA_BF16), k_buf, v_buf)
    pk, pv = synth.pin_kv(s)
    ring.pin_prefix(dev(pk), dev(pv), s.pin_tokens)
    pool = [tuple(dev(a) for a in synth.frame_kv(s, f)) for f in range(4)]
    for f in range(s.num_slots + 3):
        ring.push_frame(*pool[f % 4])
    nb = ring.capsule_bytes()
    cap = torch.empty(nb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    st = ring.snapshot(cap, stream=stream)
    ring.restore(cap, st, stream=stream)
    torch.cuda.synchronize()
    res = {"workload": "long_history_18L ring capsule", "capsule_bytes": nb, "calls": n_calls}
    for name, fn in (("snapshot", lambda: ring.snapshot(cap, stream=stream)),
                     ("restore", lambda: ring.restore(cap, st, stream=stream))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_calls):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n_calls
        res[f"{name}_us"] = round(us, 1)
        res[f"{name}_gbs"] = round(2 * nb / (us * 1e-6) / 1e9, 1)
    ring.close()
    return res


def bench_stack(args, torch, L, configs, synth, full_layer=False, shape=None):
    """Whole 18-layer denoising step, chained layer by layer, graph-replayed:
    the Pi0.5-like stack by default, or `shape` (the long-history cache with
    the same layer dims); with full_layer, every layer also runs the SwiGLU
    FFN block (its own AdaRMSNorm gamma, gate/up 1024 -> 4096, down 4096 ->
    1024)."""
    s = shape if shape is not None else (configs.PI05_18L_FFN if full_layer else configs.PI05_18L)
    dev = lambda a: torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda()  # noqa: E731
    import numpy as np
    shp = (s.num_layers, s.max_seq_len, s.n_kv_heads, s.head_dim)
    k_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
    v_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
    ring = L.Ring(L.rb_config(s.num_layers, s.n_kv_heads, s.head_dim, s.pin_tokens, s.num_slots,
                              s.tokens_per_frame, L.PA_BF16), k_buf, v_buf)
    pk, pv = synth.pin_kv(s)
    ring.pin_prefix(dev(pk), dev(pv), s.pin_tokens)
    pool = [tuple(dev(a) for a in synth.frame_kv(s, f)) for f in range(4)]
    for f in range(s.num_slots):
        ring.push_frame(*pool[f % 4])
    log("generating 18 layers of projection and gamma-MLP weights")
    pw = [synth.proj_weights(s, l) for l in range(s.num_layers)]
    wqkv = dev(np.stack([w[0] for w in pw]))
    wo = dev(np.stack([w[1] for w in pw]))
    mw = [synth.mlp_weights(s, l) for l in range(s.num_layers)]
    mlp = L.ada_mlp(*(dev(np.stack([w[i] for w in mw])) for i in range(4)), s.num_layers, s.cond_emb,
                    s.state_dim, s.hidden_dim, s.model_dim)
    ffn_keep, mlp_f, gamma_f = (None, None, None), None, None
    if full_layer:
        log("generating 18 layers of SwiGLU FFN weights")
        fw = [synth.ffn_weights(s, l) for l in range(s.num_layers)]
        ffn_keep = tuple(dev(np.stack([w[i] for w in fw])) for i in range(3))
        del fw
        mf = [synth.ffn_mlp_weights(s, l) for l in range(s.num_layers)]
        mlp_f = L.ada_mlp(*(dev(np.stack([w[i] for w in mf])) for i in range(4)), s.num_layers, s.cond_emb,
                          s.state_dim, s.hidden_dim, s.model_dim)
        gamma_f = torch.empty((s.num_layers, s.steps_per_frame, s.model_dim), dtype=torch.float32, device="cuda")
    st_plain = L.pa_stack(s.num_layers, s.n_dyn, s.model_dim, s.n_q_heads, wqkv, wo, s.eps, s.scale, 0.1, 0,
                          s.ffn_dim, *ffn_keep)

    # the product path: the same weights in the fragment-packed order
    def packed(w, n, k):
        out = torch.empty_like(w)
        L.pa_pack_weight(w, n, k, out)
        return out

    nl, hd, fd = s.num_layers, s.n_q_heads * s.head_dim, s.ffn_dim
    pk_keep = (None, None, None)
    if full_layer:
        pk_keep = (packed(ffn_keep[0], nl * fd, s.model_dim), packed(ffn_keep[1], nl * fd, s.model_dim),
                   packed(ffn_keep[2], nl * s.model_dim, fd))
    st = L.pa_stack(s.num_layers, s.n_dyn, s.model_dim, s.n_q_heads, packed(wqkv, nl * s.qkv_out, s.model_dim),
                    packed(wo, nl * s.model_dim, hd), s.eps, s.scale, 0.1, 0, s.ffn_dim, *pk_keep, packed=1)
    wsb = max(L.pa_denoise_step_workspace_bytes(ring, st), L.pa_denoise_step_workspace_bytes(ring, st_plain))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    gamma = torch.empty((s.num_layers, s.steps_per_frame, s.model_dim), dtype=torch.float32, device="cuda")
    gwsb = L.ada_gamma_workspace_bytes(mlp, s.steps_per_frame)
    gws = torch.empty(gwsb, dtype=torch.uint8, device="cuda")
    ts = [1.0 - k / s.steps_per_frame for k in range(s.steps_per_frame)]
    x = torch.empty((s.n_dyn, s.model_dim), dtype=torch.int16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_frames = args.stack_frames
    xs = dev(synth.normal((n_frames, s.n_dyn, s.model_dim), "bf16", s.cfg_id, synth.T_X, 11))
    states = dev(synth.normal((n_frames, s.state_dim), "bf16", s.cfg_id, synth.T_STATE, 11))
    state = torch.empty(s.state_dim, dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        for k in range(s.steps_per_frame):
            L.pa_denoise_step(ring, st, x, gamma[:, k], s.steps_per_frame * s.model_dim, flag, ws, wsb,
                              gamma_ffn=None if gamma_f is None else gamma_f[:, k])
    g_plain = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_plain, stream=side):
        for k in range(s.steps_per_frame):
            L.pa_denoise_step(ring, st_plain, x, gamma[:, k], s.steps_per_frame * s.model_dim, flag, ws, wsb,
                              gamma_ffn=None if gamma_f is None else gamma_f[:, k])

    def frame(i):
        ring.push_frame(*pool[i % 4])
        state.copy_(states[i % n_frames])
        L.ada_gamma(mlp, ts, state, gamma, gws, gwsb)
        if mlp_f is not None:
            L.ada_gamma(mlp_f, ts, state, gamma_f, gws, gwsb)
        x.copy_(xs[i % n_frames])
        g.replay()

    settle(torch, args.settle_ms, frame, 2)
    for i in range(2):
        frame(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_frames):
        frame(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # the ten steps alone (graph replays back to back, no push / gamma)
    t1 = time.perf_counter()
    for i in range(n_frames):
        g.replay()
    torch.cuda.synchronize()
    el_steps = time.perf_counter() - t1
    # the same ten steps on the unpacked (nn.Linear layout) weights
    g_plain.replay()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(n_frames):
        g_plain.replay()
    torch.cuda.synchronize()
    el_plain = time.perf_counter() - t2
    ring.close()
    return {
        "workload": s.name,
        "us_per_step": el_steps / (n_frames * s.steps_per_frame) * 1e6,
        "weights": "fragment-packed (pa_pack_weight)",
        "us_per_step_unpacked_weights": el_plain / (n_frames * s.steps_per_frame) * 1e6,
        "steps_per_s": n_frames * s.steps_per_frame / el_steps,
        "frames_per_s_incl_push_gamma": n_frames / el,
        "us_per_frame_incl_push_gamma": el / n_frames * 1e6,
        "frames_timed": n_frames,
        "nonfinite_flag": int(flag.item()),
        "config": {"layers": s.num_layers, "model_dim": s.model_dim, "q_heads": s.n_q_heads,
                   "kv_heads": s.n_kv_heads, "head_dim": s.head_dim, "pin_tokens": s.pin_tokens,
                   "window": f"{s.num_slots}x{s.tokens_per_frame}", "suffix": s.n_dyn,
                   "steps_per_frame": s.steps_per_frame, "ffn": f"SwiGLU {s.ffn_dim}" if s.ffn_dim else "none"},
    }


def bench_shared_kv(args, torch, L, configs, synth, budgets=(1, 5, 10), n_frames=20):
    """Shared-KV multi-reader frames: the long-history cache read by the action
    suffix (10 denoising steps, 18 layers) and by 16 decode streams, one query
    token each, advancing k decode steps per frame (k swept over `budgets`).
    Private tails start staggered at 2j mod 30 tokens, grow by one token per
    decode step, and a stream whose tail reaches 30 tokens retires: its next
    token starts a new request."""
    import numpy as np
    s = configs.SHARED_KV
    dev = lambda a: torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda()  # noqa: E731
    shp = (s.num_layers, s.max_seq_len, s.n_kv_heads, s.head_dim)
    k_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
    v_buf = torch.zeros(shp, dtype=torch.int16, device="cuda")
    ring = L.Ring(L.rb_config(s.num_layers, s.n_kv_heads, s.head_dim, s.pin_tokens, s.num_slots,
                              s.tokens_per_frame, L.PA_BF16), k_buf, v_buf)
    pk, pv = synth.pin_kv(s)
    ring.pin_prefix(dev(pk), dev(pv), s.pin_tokens)
    pool = [tuple(dev(a) for a in synth.frame_kv(s, f)) for f in range(4)]
    for f in range(s.num_slots):
        ring.push_frame(*pool[f % 4])
    steps_in = [tuple(dev(a) for a in synth.suffix_qkv(s, 0, k)) for k in range(s.steps_per_frame)]
    a_args = L.pattn_args(0, s.num_layers, s.n_q_heads, s.n_dyn, s.scale, L.PA_BF16)
    a_wsb = L.pattn_workspace_bytes(ring, a_args)
    a_ws = torch.empty(a_wsb, dtype=torch.uint8, device="cuda")
    a_out = torch.empty((s.num_layers, s.n_dyn, s.n_q_heads, s.head_dim), dtype=torch.int16, device="cuda")
    G, cap = s.n_streams, s.tail_capacity
    d_args = L.decode_args(0, s.num_layers, s.n_q_heads, G, cap, s.scale, L.PA_BF16, 0, 1)
    d_wsb = L.pattn_decode_workspace_bytes(ring, d_args)
    d_ws = torch.empty(d_wsb, dtype=torch.uint8, device="cuda")
    tail_k = torch.zeros((s.num_layers, G, cap, s.n_kv_heads, s.head_dim), dtype=torch.int16, device="cuda")
    tail_v = torch.zeros_like(tail_k)
    dq = [dev(synth.decode_q(s, 0, t)) for t in range(2)]
    dkv = [tuple(dev(a) for a in synth.decode_kv(s, 0, t)) for t in range(2)]
    d_out = torch.empty((s.num_layers, G, s.n_q_heads, s.head_dim), dtype=torch.int16, device="cuda")
    ovf = torch.zeros(1, dtype=torch.int32, device="cuda")

    f_wsb = L.pattn_fused_workspace_bytes(ring, a_args, d_args)
    f_ws = torch.empty(f_wsb, dtype=torch.uint8, device="cuda")

    def frame(i, k_dec, ev=None):
        ring.push_frame(*pool[i % 4])
        for k in range(s.steps_per_frame):
            L.pattn_step(ring, a_args, *steps_in[k], a_out, a_ws, a_wsb)
        if ev is not None:
            ev[0].record()
        for t in range(k_dec):
            L.pattn_append_private(ring, d_args, tail_k, tail_v, tail_len, *dkv[t % 2], ovf)
            L.pattn_decode(ring, d_args, dq[t % 2], tail_k, tail_v, tail_len, d_out, d_ws, d_wsb)
        if ev is not None:
            ev[1].record()

    def frame_fused(i, k_dec, ev=None):
        # decode step t rides on action step t: one pass over the shared cache for both
        ring.push_frame(*pool[i % 4])
        for k in range(s.steps_per_frame):
            if k < k_dec:
                L.pattn_append_private(ring, d_args, tail_k, tail_v, tail_len, *dkv[k % 2], ovf)
                L.pattn_fused_step(ring, a_args, *steps_in[k], a_out, d_args, dq[k % 2], tail_k, tail_v, tail_len,
                                   d_out, f_ws, f_wsb)
            else:
                L.pattn_step(ring, a_args, *steps_in[k], a_out, a_ws, a_wsb)

    tail_len = dev(np.array([(2 * j) % cap for j in range(G)], dtype=np.int32))
    settle(torch, args.settle_ms, lambda i: frame_fused(i, 1), 10)
    sweep, sweep_fused = {}, {}
    for k_dec in budgets:
        tail_len = dev(np.array([(2 * j) % cap for j in range(G)], dtype=np.int32))
        frame(0, k_dec)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_frames)]
        t0 = time.perf_counter()
        for i in range(n_frames):
            frame(1 + i, k_dec, evs[i])
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        dec_us = sum(a.elapsed_time(b) for a, b in evs) / n_frames * 1e3 / k_dec
        assert int(ovf.item()) == 0, "a private tail overflowed with retiring on"
        sweep[k_dec] = {"frames_per_s": n_frames / el, "decode_tokens_per_s": G * k_dec * n_frames / el,
                        "decode_step_us": dec_us, "frames_timed": n_frames}
        if k_dec <= s.steps_per_frame:
            tail_len = dev(np.array([(2 * j) % cap for j in range(G)], dtype=np.int32))
            frame_fused(0, k_dec)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(n_frames):
                frame_fused(1 + i, k_dec)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            assert int(ovf.item()) == 0, "a private tail overflowed with retiring on"
            sweep_fused[k_dec] = {"frames_per_s": n_frames / el, "decode_tokens_per_s": G * k_dec * n_frames / el,
                                  "frames_timed": n_frames}
    ring.close()
    k1, f1 = sweep[budgets[0]], sweep_fused[budgets[0]]
    # The frame loop reported first is the fused one (decode step k rides on
    # action step k: one pass over the shared cache for both); the loop with
    # separate passes is reported beside it, with its decode step time.
    return {"workload": "shared_kv_multitask", "loop": "fused action + decode pass",
            "frames_per_s": f1["frames_per_s"], "decode_tokens_per_s": f1["decode_tokens_per_s"],
            "frames_per_s_separate_passes": k1["frames_per_s"], "decode_step_us": k1["decode_step_us"],
            "frames_timed": n_frames, "decode_budget_sweep": {f"k={k}": v for k, v in sweep.items()},
            "fused_decode_budget_sweep": {f"k={k}": v for k, v in sweep_fused.items()},
            "config": {"layers": 18, "cache": "256 + 8x768", "action_suffix": 51, "steps_per_frame": 10,
                       "decode_streams": G, "tail_capacity": cap, "retire_at": cap,
                       "decode_steps_per_frame": budgets[0]}}


def cpu_baseline(budget_s):
    """Time the float64 CPU oracle on bounded samples of three workloads: the
    long-history 18-layer attention step (the headline), the Pi0.5-like
    single-layer attention step, and the Pi0.5-like 18-layer stack step
    (norm, QKV, attention, out-projection per layer, then the Euler update).
    Each gets its share of budget_s; the long-history step is also timed on
    one BLAS thread."""
    import numpy as np
    from oracle.attention import full_attention
    from oracle import stack as ostack
    from partitioned_kv_cache_amd import configs, synth

    def attention_ctx(s):
        pk, pv = synth.pin_kv(s)
        frames = [synth.frame_kv(s, f % 4) for f in range(s.num_slots)]
        q, kd, vd = synth.suffix_qkv(s, 0, 0)
        ctx = []
        for l in range(s.num_layers):
            ck = np.concatenate([synth.widen(pk[l])] + [synth.widen(f[0][l]) for f in frames] + [synth.widen(kd[l])])
            cv = np.concatenate([synth.widen(pv[l])] + [synth.widen(f[1][l]) for f in frames] + [synth.widen(vd[l])])
            ctx.append((synth.widen(q[l]), ck, cv))
        return ctx

    def timed_layers(s, ctx, budget):
        done = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 <= budget:
            l = done % s.num_layers
            full_attention(ctx[l][0], ctx[l][1], ctx[l][2], s.scale)
            done += 1
        return done, time.perf_counter() - t0

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    cpu = _cpu_model()
    # the headline: long-history 18-layer attention step
    s4 = configs.LONG_18L
    ctx4 = attention_ctx(s4)
    n4, el4 = timed_layers(s4, ctx4, budget_s * 0.45)
    res = {"value": n4 / s4.num_layers / el4, "unit": "denoise steps/s", "cores": threads, "kind": "oracle",
           "sample": f"long-history 18-layer attention step: {n4} layer-attentions ({n4 / s4.num_layers:.2f} steps) "
                     f"of frame 0 step 0, float64 NumPy, {el4:.1f} s; cpu: {cpu}; "
                     f"{len(os.sched_getaffinity(0))} host threads available"}
    if threadpool_limits is not None:
        with threadpool_limits(1):
            n1, el1 = timed_layers(s4, ctx4, budget_s * 0.15)
        res["value_1_thread"] = n1 / s4.num_layers / el1
        res["sample_1_thread"] = f"{n1} layer-attentions of the long-history step, one BLAS thread, {el1:.1f} s"
    del ctx4
    # Pi0.5-like single-layer attention step
    s2 = configs.PI05_1L
    ctx2 = attention_ctx(s2)
    n2, el2 = timed_layers(s2, ctx2, budget_s * 0.15)
    res["pi05_like_1L"] = {"steps_per_s": n2 / el2, "sample": f"{n2} single-layer steps, {el2:.1f} s"}
    # Pi0.5-like 18-layer stack step (the whole chained step, gamma given)
    s3 = configs.PI05_18L
    pk, pv = synth.pin_kv(s3)
    frames = [synth.frame_kv(s3, f) for f in range(s3.num_slots)]
    caches_k = [np.concatenate([synth.widen(pk[l])] + [synth.widen(f[0][l]) for f in frames])
                for l in range(s3.num_layers)]
    caches_v = [np.concatenate([synth.widen(pv[l])] + [synth.widen(f[1][l]) for f in frames])
                for l in range(s3.num_layers)]
    pw = [synth.proj_weights(s3, l) for l in range(s3.num_layers)]
    wq, wo = [synth.widen(w[0]) for w in pw], [synth.widen(w[1]) for w in pw]
    gam = [np.ones(s3.model_dim)] * s3.num_layers
    x = synth.widen(synth.flow_x(s3, 0))
    n3 = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 <= budget_s * 0.25 or n3 == 0:
        x, _ = ostack.denoise_step(x, gam, s3.eps, wq, wo, caches_k, caches_v, s3.scale, s3.n_q_heads,
                                   s3.n_kv_heads, s3.head_dim)
        n3 += 1
    el3 = time.perf_counter() - t0
    res["pi05_like_18L_stack_step"] = {"steps_per_s": n3 / el3, "us_per_step": el3 / n3 * 1e6,
                                       "sample": f"{n3} chained 18-layer steps, {el3:.1f} s"}
    return res


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "partial_mfma_long_history_traffic.md")
KERNEL_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "partitioned_kv_cache_amd", "csrc",
                             "attention.hip")


def stored_traffic():
    """HBM bytes per launch of the partial kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's readings), or
    None when the summary is missing or the kernel source changed since."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(l.split(":", 1) for l in text.splitlines() if l.startswith(("source_sha256:", "traffic_bytes:")))
    if fields.get("source_sha256", "").strip() != src:
        return None
    try:
        return int(float(fields["traffic_bytes"].strip()))
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, mb):
    """A plain device copy of known size, for scaling the traffic counters."""
    n = mb * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, plus family, model
    and stepping (a virtualised host may report only a short model name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v
            if not line.strip() and fields:
                break
    except OSError:
        pass
    if not fields:
        return "unknown"
    return (f"{fields.get('model name', '?')} (family {fields.get('cpu family', '?')}, model "
            f"{fields.get('model', '?')}, stepping {fields.get('stepping', '?')})")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--splits", type=int, default=0, help="KV splits per layer (0 = library default)")
    ap.add_argument("--stack-frames", type=int, default=50)
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-shared", action="store_true", help="skip the shared-KV multi-reader frame")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--headline-only", action="store_true",
                    help="run only the cold-MALL headline step (for profiler passes)")
    ap.add_argument("--cold-rings", type=int, default=3,
                    help="independent rings served round-robin for the cold-MALL headline (3 x 118 MB > 256 MB)")
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="untimed run of each workload's own loop before its warmup steps (0 = none)")
    ap.add_argument("--kernel-launches", type=int, default=30,
                    help="partial-kernel launches timed one by one for the roofline (at least 20)")
    ap.add_argument("--no-fp32-partials", action="store_true",
                    help="skip the headline variant with FP32 split partials")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB MiB five times (traffic-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path is built for a "
              "single MI355X; nothing here shards across GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch
    from partitioned_kv_cache_amd import _lib as L, configs, synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    if args.headline_only:
        args.no_stack = args.no_shared = True
        args.cpu_budget = 0
    lh = bench_long_history(args, torch, L, configs, synth, n_rings=args.cold_rings)
    log(f"long history, cold MALL ({args.cold_rings} rings): {lh['steps_per_s']:.1f} steps/s, partial kernel "
        f"{lh['partial_us']:.1f} us ({lh['partial_tflops']:.0f} TFLOP/s, {lh['partial_gbs']:.0f} GB/s)")
    lh_op = bench_long_history(args, torch, L, configs, synth, n_rings=args.cold_rings, q_layout=L.PA_Q_OPERAND)
    log(f"long history, cold MALL, Q in operand order: {lh_op['steps_per_s']:.1f} steps/s, partial kernel "
        f"{lh_op['partial_us']:.1f} us")
    lh_f32 = None
    if not args.headline_only and not args.no_fp32_partials:
        lh_f32 = bench_long_history(args, torch, L, configs, synth, n_rings=args.cold_rings, partials_f32=1)
        log(f"long history, cold MALL, FP32 partials: {lh_f32['steps_per_s']:.1f} steps/s, partial kernel "
            f"{lh_f32['partial_us']:.1f} us")
    warm = small = async_push = ada_qkv = capsule = None
    if not args.headline_only:
        warm = bench_long_history(args, torch, L, configs, synth, n_rings=1)
        log(f"long history, warm MALL: {warm['steps_per_s']:.1f} steps/s, partial kernel {warm['partial_us']:.1f} us")
        small = [bench_small(args, torch, L, c) for c in (configs.TINY, configs.PI05_1L)]
        for sm in small:
            log(f"{sm['workload']}: {sm['us_per_call']:.1f} us per call eager, {sm['us_per_call_graph']:.1f} in a graph")
        ada_qkv = bench_adanorm_qkv(args, torch, L, configs, synth)
        log(f"ada_rmsnorm_qkv: {ada_qkv['us_per_call']:.1f} us per call eager, {ada_qkv['us_per_call_graph']:.1f} "
            f"in a graph ({ada_qkv['gbs_graph']:.0f} GB/s)")
        capsule = bench_capsule(args, torch, L, configs, synth)
        log(f"capsule ({capsule['capsule_bytes'] / 1e6:.1f} MB): snapshot {capsule['snapshot_us']:.1f} us "
            f"({capsule['snapshot_gbs']:.0f} GB/s), restore {capsule['restore_us']:.1f} us")
        async_push = bench_async_push(args, torch, L, configs, synth)
        log(f"async push: {async_push['frames_per_s_sync_push']:.1f} frames/s synchronous, "
            f"{async_push['frames_per_s_overlapped_push']:.1f} overlapped")
    stack = full = chained = None
    if not args.no_stack:
        chained = bench_stack(args, torch, L, configs, synth, shape=configs.LONG_18L_FULL)
        log(f"long history chained 18-layer denoise step: {chained['us_per_step']:.1f} us/step")
        stack = bench_stack(args, torch, L, configs, synth)
        log(f"pi05 18L stack: {stack['us_per_step']:.1f} us/step")
        full = bench_stack(args, torch, L, configs, synth, full_layer=True)
        log(f"pi05 18L full layer (with SwiGLU FFN): {full['us_per_step']:.1f} us/step")
    shared = None
    if not args.no_shared:
        shared = bench_shared_kv(args, torch, L, configs, synth)
        log(f"shared KV: {shared['frames_per_s']:.1f} frames/s fused ({shared['frames_per_s_separate_passes']:.1f} "
            f"with separate passes, decode step {shared['decode_step_us']:.1f} us)")
    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(args.cpu_budget)
        log(f"cpu oracle: {cpu['value']:.4f} steps/s on {cpu['cores']} threads")
    s = configs.LONG_18L
    line = {
        "metric": METRIC,
        "value": lh["steps_per_s"],
        "unit": "denoise steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": lh["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded N(0,1) K/V/Q, resident in HBM; {lh['rings']} rings served round-robin, "
                "so K/V streams from HBM, not the MALL)",
        "config": {"workload": "long_history_18L", "step": "layer-batched partitioned attention: all 18 layers' "
                   "split-KV partials in one launch, then the log-sum-exp combine (every layer's suffix Q/K/V "
                   "given); a frame push before every 10th step of each ring",
                   "layers": s.num_layers, "q_heads": s.n_q_heads,
                   "kv_heads": s.n_kv_heads, "head_dim": s.head_dim, "pin_tokens": s.pin_tokens,
                   "window": f"{s.num_slots}x{s.tokens_per_frame}", "suffix": s.n_dyn,
                   "steps_per_frame": s.steps_per_frame, "kv_splits": lh["splits"] or "default",
                   "rings": lh["rings"], "mall": "cold", "pushes_timed": lh["pushes_timed"],
                   "settle": {"ms": args.settle_ms, "steps": lh["settle_steps"],
                              "what": "the same step loop run untimed before the warmup steps (matrix-core kernels "
                                      "run slower for their first few hundred launches after the GPU idles)",
                              "partial_us_first_100_launches": None if lh["first_launches_us"] is None
                              else round(lh["first_launches_us"], 3)}},
        # frames/s = 1 / (t_push + 10 t_step): the timed steps include their
        # pushes (one per 10 steps of each ring), so this is steps/s / 10; the
        # push alone and the step without its share of pushes are timed beside it
        "frames_per_s": lh["steps_per_s"] / s.steps_per_frame,
        "push_us": round(lh["push_us"], 2),
        "step_us_excl_push": round(lh["ms_per_step"] * 1e3 - lh["pushes_timed"] / max(args.steps, 1) * lh["push_us"],
                                   2),
        "roofline": {"bound": "mfma", "achieved": round(lh["partial_tflops"], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(lh["partial_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(), "kernel": "partial_mfma<256>",
                     "kernel_us": round(lh["partial_us"], 3), "kernel_us_sd": round(lh["partial_us_sd"], 3),
                     "kernel_us_min": round(lh["partial_us_min"], 3), "kernel_us_max": round(lh["partial_us_max"], 3),
                     "timed_launches": lh["timed_launches"],
                     "flops_per_launch": lh["flops"], "algo_bytes_per_launch": lh["algo_bytes"]},
        "hbm": {"achieved": round(lh["partial_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(lh["partial_gbs"] / HBM_PEAK_GBS, 4),
                "kv_stream_gbs_whole_step": round(lh["kv_gbs_step"], 1)},
        "cpu_baseline": cpu,
        # the same cold step with Q already in the kernel's operand order
        # (PA_Q_OPERAND): what a producer that writes Q in that order gets
        "cold_q_operand_order": {"steps_per_s": lh_op["steps_per_s"], "ms_per_step": lh_op["ms_per_step"],
                                 "partial_us": round(lh_op["partial_us"], 3),
                                 "partial_tflops": round(lh_op["partial_tflops"], 2),
                                 "frac": round(lh_op["partial_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    if lh_f32 is not None:
        # the same cold step with the split partials' accumulator kept in FP32
        # (pattn_args.partials_f32 = 1) instead of bf16
        line["cold_fp32_partials"] = {"steps_per_s": lh_f32["steps_per_s"], "ms_per_step": lh_f32["ms_per_step"],
                                      "partial_us": round(lh_f32["partial_us"], 3),
                                      "partial_tflops": round(lh_f32["partial_tflops"], 2),
                                      "frac": round(lh_f32["partial_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)}
    if chained is not None:
        line["long_history_18L_chained_step"] = chained
    if warm is not None:
        line["warm_mall"] = {"rings": 1, "steps_per_s": warm["steps_per_s"], "ms_per_step": warm["ms_per_step"],
                             "partial_us": round(warm["partial_us"], 3),
                             "partial_tflops": round(warm["partial_tflops"], 2),
                             "kv_stream_gbs_whole_step": round(warm["kv_gbs_step"], 1)}
    if small is not None:
        line["small_configs"] = {sm["workload"]: {"us_per_call": round(sm["us_per_call"], 2),
                                                  "us_per_call_graph": round(sm["us_per_call_graph"], 2),
                                                  "calls": sm["calls"], "layers": sm["layers"],
                                                  "cached_tokens": sm["cached_tokens"], "suffix": sm["suffix"]}
                                 for sm in small}
    if ada_qkv is not None:
        line["adarmsnorm_qkv"] = ada_qkv
    if capsule is not None:
        line["ring_capsule"] = capsule
    if async_push is not None:
        line["async_push"] = async_push
    if stack is not None:
        line["pi05_18L_full_step"] = stack
        line["pi05_18L_full_layer_step"] = full
    if shared is not None:
        line["shared_kv_multitask"] = shared
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
