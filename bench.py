#!/usr/bin/env python3
"""Draft + verify cycles per second on one MI355X.

One step = one whole cycle of the hot path on one batch:
    len[b] <- C_b (hold the context at the workload's length, a D2D copy)
    dflash_inject_kv   (features of the tau_b rows accepted last cycle)
    dflash_draft_block (anchor + gamma-1 masks -> gamma-1 draft tokens)
    dflash_verify      (against planted target tokens -> tau_b, next anchor)
Inputs are seeded synthetic tensors already resident in HBM.  The target's own
forward pass is outside the cycle: its outputs (the features of accepted rows
and its greedy tokens at the block positions) are synthetic inputs, planted so
that each cycle accepts a truncated-geometric number of drafts (mean ~6 at
gamma 16).  Drafting is deterministic, so an untimed planning pass records the
drafts of every cycle and builds the target tokens; the timed pass replays the
identical sequence and must reproduce every planted accept length.

Prints one JSON line.  `roofline` is for the dominant kernel (the fused final
norm + LM head + argmax launch), timed per launch with HIP events recorded by
the library around that launch in traced cycles of the same workload;
`cycle_roofline` (and `hbm_roofline_frac`) is the whole cycle's fraction.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft+verify cycles/sec and % HBM roofline, Qwen3-8B shape, gamma=16"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Hip:
    """Minimal ctypes access to HIP events (the library records them)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        assert self.h.hipEventSynchronize(b) == 0
        assert self.h.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def destroy(self, e):
        self.h.hipEventDestroy(e)


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(HERE, "profiles", "lm_head_argmax_qwen3_8b_b1_traffic.md")


def kernel_fingerprint() -> str:
    """SHA-256 prefix of the sources that decide what the LM-head kernel reads:
    csrc/common.hpp, csrc/gemm.hpp and the plan_gemm function of csrc/dflash.hip."""
    csrc = os.path.join(HERE, "block_diffusion_drafter_states_amd", "csrc")
    h = hashlib.sha256()
    for f in ("common.hpp", "gemm.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(csrc, "dflash.hip")) as fh:
        src = fh.read()
    i = src.index("GemmPlan plan_gemm(")
    h.update(src[i:src.index("\n}\n", i)].encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_is_profiled: bool):
    """HBM bytes per LM-head launch from the committed rocprofv3 counter summary,
    or None when the workload differs or the kernel sources changed since."""
    if not workload_is_profiled or not os.path.exists(TRAFFIC_PROFILE):
        return None
    with open(TRAFFIC_PROFILE) as fh:
        for line in fh:
            if line.startswith("traffic-record:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("source_fingerprint") == kernel_fingerprint():
                    return int(rec["bytes_per_launch"])
    return None


SHAPES = {"tiny_f32": "tiny fp32 drafter", "qwen3_4b_drafter": "Qwen3-4B-shaped drafter (tied LM head)",
          "qwen3_8b_drafter": "Qwen3-8B-shaped drafter", "llama31_8b_drafter_b32": "LLaMA-3.1-8B-shaped drafter",
          "coder30b_drafter_longctx": "Qwen3-Coder-30B-drafter-shaped (GQA 8)"}
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}     # dense, MI355X published
N_CU, CLOCK_HZ = 256, 2.4e9                           # MI355X compute units and peak engine clock


def gemm_flops(cfg, B, gamma, tau_mean):
    """Multiply-add flops of the cycle's projections (2 per MAC): injection of tau rows per
    sequence, the drafter's projections over the B * gamma block rows, the LM head over all of
    them (the kernel computes the anchor row too)."""
    H, F, D, L = cfg.hidden, cfg.n_feat, cfg.head_dim, cfg.n_layers
    rows_inj, rows_blk = B * tau_mean, B * gamma
    inj = rows_inj * (F * H * H + L * 2 * cfg.n_kv * D * H)
    blk = rows_blk * L * ((cfg.n_q + 2 * cfg.n_kv) * D * H + cfg.n_q * D * H + 3 * cfg.inter * H)
    lm = rows_blk * cfg.vocab * H
    return 2.0 * (inj + blk + lm)


def algorithmic_bytes(cfg, B, C_mean, tau_mean):
    """Bytes one cycle must move: each weight once (W_k/W_v once for injection and
    drafting together), the context K/V once, feature rows read, new K/V written."""
    e = cfg.elem_bytes
    H, F, D, L = cfg.hidden, cfg.n_feat, cfg.head_dim, cfg.n_layers
    parts = {
        "w_fuse": H * F * H * e,
        "w_k_w_v": L * 2 * cfg.n_kv * D * H * e,
        "w_q_w_o": L * 2 * cfg.n_q * D * H * e,
        "mlp": L * 3 * cfg.inter * H * e,
        "lm_head": cfg.vocab * H * e,
        "ctx_kv": L * B * cfg.n_kv * C_mean * D * 2 * e,
        "features_kv_rows": B * tau_mean * (F * H + L * 2 * cfg.n_kv * D) * e,
    }
    return parts, sum(parts.values())


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_baseline(cfg, W, K, V, lengths, feats, anchors, plant_k, gammas, budget_s):
    """The oracle on a bounded sample of the same workload (block size of cycle n:
    gammas[n % len(gammas)]), in its fp32 mode (DraftModel / KVCache dtype float32: numpy
    fp32 BLAS, the same bf16 rounding points), timed once with every BLAS thread the host
    gives it and once with one thread: the median cycle time of the cycles after 1 warm-up
    that fit the time budget (at least one)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import dflash as O
    from synth import gen

    t0 = time.time()
    m = O.DraftModel(cfg, W, dtype=np.float32)
    kv = O.KVCache.from_storage(cfg, K, V, lengths, dtype=np.float32)
    log(f"oracle set-up {time.time() - t0:.1f}s")
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    B = len(lengths)

    def run(budget):
        tau = [int(k) + 1 for k in plant_k[0]]
        anchor = [int(a) for a in anchors]
        times = []
        n = 0
        start = time.time()
        while True:
            c0 = time.time()
            for b in range(B):
                kv.len[b] = lengths[b]
                f = O.decode_storage(feats[n % len(feats)][b, : tau[b]], np.float32)
                O.inject(m, kv, b, f)
                d = O.draft(m, kv, b, anchor[b], gammas[n % len(gammas)])
                y = gen.planted_targets(cfg, d[None, :], np.array([plant_k[n % len(plant_k)][b]]),
                                        tag=f"cpu.{n}.{b}")[0]
                t, _, nxt = O.verify(d, y)
                tau[b], anchor[b] = t, nxt
            times.append(time.time() - c0)
            n += 1
            if n >= 2 and time.time() - start >= budget:
                break
        timed = times[1:] if len(times) > 1 else times     # the first cycle is the warm-up
        return statistics.median(timed), len(timed)

    s_all, n_all = run(budget_s)
    with threadpool_limits(limits=1, user_api="blas"):
        s_one, n_one = run(budget_s)
    log(f"oracle cycle {s_all:.3f}s ({threads} BLAS threads), {s_one:.3f}s (1 thread)")
    return {"value": round(1.0 / s_all, 4), "unit": "cycles/s", "cores": int(threads), "kind": "oracle",
            "value_1_core": round(1.0 / s_one, 4), "cpu_model": _cpu_model(), "blas_threads": int(threads),
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"whole cycles (inject the accepted rows + draft + verify) of the same workload, batch {B}; "
                      f"oracle in its fp32 mode (numpy float32 BLAS, bf16 rounding points kept); median of "
                      f"{n_all} timed cycles after 1 warm-up with {threads} BLAS threads, and of {n_one} with 1"}


GEMM_LAUNCHES = ("fuse", "inject_kv", "qkv_proj", "o_proj", "gate_up", "down_proj", "lm_head_argmax")


def measured_peaks(torch):
    """What plain probe kernels reach on this GPU (libdflash_probe.so): the HBM read rate of a
    grid-stride streaming kernel over 4 GiB (plain loads, 16 workgroups per CU; and with the
    non-temporal hint, eight loads in flight per thread, one workgroup per CU) and the bf16 MFMA
    rate of independent 16x16x32 and 32x32x16 MFMA chains on every SIMD (each the median of 5)."""
    lib = ctypes.CDLL(os.path.join(HERE, "block_diffusion_drafter_states_amd", "libdflash_probe.so"))
    lib.dflash_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    lib.dflash_probe_read_nt.argtypes = lib.dflash_probe_read.argtypes
    lib.dflash_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.dflash_probe_mfma32.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = 4 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    blocks = 256 * 16
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    fsink = torch.zeros(blocks, dtype=torch.float32, device="cuda")

    def time_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if fn() != 0:
            raise RuntimeError("probe launch failed")
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    read = lambda: lib.dflash_probe_read(buf.data_ptr(), nbytes, 0x9E3779B9, sink.data_ptr(), blocks, stream)
    time_ms(read)
    gbs = nbytes / (statistics.median(time_ms(read) for _ in range(5)) * 1e-3) / 1e9
    read_nt = lambda: lib.dflash_probe_read_nt(buf.data_ptr(), nbytes, 0x9E3779B9, sink.data_ptr(), 256, stream)
    time_ms(read_nt)
    gbs_nt = nbytes / (statistics.median(time_ms(read_nt) for _ in range(5)) * 1e-3) / 1e9
    iters, mblocks = 2000, 256 * 8
    mfma = lambda: lib.dflash_probe_mfma(iters, mblocks, fsink.data_ptr(), stream)
    time_ms(mfma)
    flops = mblocks * 4 * iters * 8 * 16384.0
    tflops = flops / (statistics.median(time_ms(mfma) for _ in range(5)) * 1e-3) / 1e12
    mfma32 = lambda: lib.dflash_probe_mfma32(iters, mblocks, fsink.data_ptr(), stream)
    time_ms(mfma32)
    flops32 = mblocks * 4 * iters * 4 * 32768.0
    tflops32 = flops32 / (statistics.median(time_ms(mfma32) for _ in range(5)) * 1e-3) / 1e12
    del buf
    torch.cuda.empty_cache()
    return {"read_GBs": round(gbs, 1), "read_nt_GBs": round(gbs_nt, 1), "mfma_bf16_TFLOPs": round(tflops, 1),
            "mfma32_bf16_TFLOPs": round(tflops32, 1)}


def prefill(args, dfl, cfg, gen, torch):
    """Injection of a whole prompt's feature rows (C3: 4096 positions) into an empty cache:
    the fusion and every layer's W_k | W_v over all rows, an MFMA-bound contraction."""
    B, rows = 1, cfg.ctx
    cap = (rows + 2 * cfg.gamma_max + 63) // 64 * 64
    W = gen.weights(cfg)
    model = dfl.Model(cfg, W, device="cuda", max_batch=B, kv_capacity=cap)
    cache = dfl.Cache(model)
    ws = dfl.Workspace(model, B, rows)
    feat = dfl.to_device(gen.features(cfg, B, rows, tag="bench.prefill"), "cuda")
    n_new = torch.full((B,), rows, dtype=torch.int32, device="cuda")
    times = []
    for r in range(args.warmup + args.steps):
        cache.len.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dfl.inject_kv(model, cache, feat, n_new, ws)
        e1.record()
        torch.cuda.synchronize()
        if r >= args.warmup:
            times.append(e0.elapsed_time(e1))
    assert int(cache.status.item()) == 0 and int(cache.len[0].item()) == rows
    ms = statistics.median(times)
    H, F, D, L = cfg.hidden, cfg.n_feat, cfg.head_dim, cfg.n_layers
    flops = 2.0 * rows * (F * H * H + L * 2 * cfg.n_kv * D * H)
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    tflops = flops / (ms * 1e-3) / 1e12
    print(json.dumps({"metric": "prefill injection time", "value": round(ms * 1000, 1), "unit": "us",
                      "higher_is_better": False, "steps": args.steps, "warmup": args.warmup, "dtype": cfg.dtype,
                      "config": {"workload": f"{cfg.name}: {SHAPES.get(cfg.name, cfg.name)}, "
                                             f"{rows} feature rows into an empty cache", "rows": rows},
                      "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                                   "frac": round(tflops / peak, 4), "gflop": round(flops / 1e9, 1)}}), flush=True)


def block_loss_leg(args, dfl, cfg, gen, torch):
    """The drafter's training objective over one batch of blocks (position-weighted block
    cross-entropy): the drafting forward pass with a log-sum-exp LM-head epilogue instead of
    the argmax, timed beside the drafting pass itself on the same inputs."""
    B, gamma = args.batch, cfg.gamma
    cfg = cfg.with_(batch=B)
    lengths = gen.context_lengths(cfg)
    cap = (int(lengths.max()) + 2 * cfg.gamma_max + 63) // 64 * 64
    W = gen.weights(cfg)
    model = dfl.Model(cfg, W, device="cuda", max_batch=B, kv_capacity=cap)
    cache = dfl.Cache(model)
    Kc, Vc = gen.context_kv(cfg, lengths, int(lengths.max()), tag="bench.ctx")
    cache.set_context(Kc, Vc, lengths)
    ws = dfl.Workspace(model, B, gamma)
    anchor = torch.as_tensor(gen.tokens(cfg, "bench.loss.anchor", (B,)), device="cuda")
    labels = torch.as_tensor(gen.tokens(cfg, "bench.loss.labels", (B, gamma - 1)), device="cuda")
    loss = torch.zeros((1,), dtype=torch.float32, device="cuda")
    draft = torch.zeros((B, gamma - 1), dtype=torch.int32, device="cuda")

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / args.steps

    us_loss = timed(lambda: dfl.block_loss(model, cache, gamma, anchor, labels, loss, ws))
    dz = torch.empty((B, gamma - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    us_grad = timed(lambda: dfl.block_loss(model, cache, gamma, anchor, labels, loss, ws, dlogits=dz))
    us_draft = timed(lambda: dfl.draft_block(model, cache, gamma, anchor, draft, ws))
    assert int(cache.status.item()) == 0 and math.isfinite(float(loss.item()))
    print(json.dumps({"metric": "block loss evaluations/s", "value": round(1e6 / us_loss, 2), "unit": "blocks-batches/s",
                      "higher_is_better": True, "steps": args.steps, "warmup": args.warmup, "dtype": cfg.dtype,
                      "us_per_call": round(us_loss, 1), "with_dlogits_us_per_call": round(us_grad, 1),
                      "draft_block_us_per_call": round(us_draft, 1),
                      "loss": float(loss.item()),
                      "config": {"workload": f"{cfg.name}: {SHAPES.get(cfg.name, cfg.name)}, batch {B}, gamma {gamma}, "
                                             f"context {int(lengths.mean())}", "batch": B, "gamma": gamma}}),
          flush=True)


def input_fusion_leg(args, dfl, cfg, gen, torch):
    """Cost of the two ways to condition the drafter on the target's context features, each
    followed by the drafting pass: KV injection (the fused feature through every layer's W_k /
    W_v) and input fusion (the fused feature as the input of the whole layer stack, causal over
    the new rows).  Same inputs; the context is held at its configured length."""
    import numpy as np
    B, gamma = args.batch, cfg.gamma
    cfg = cfg.with_(batch=B)
    lengths = gen.context_lengths(cfg)
    cap = (int(lengths.max()) + 2 * cfg.gamma_max + 63) // 64 * 64
    W = gen.weights(cfg)
    model = dfl.Model(cfg, W, device="cuda", max_batch=B, kv_capacity=cap)
    cache = dfl.Cache(model)
    Kc, Vc = gen.context_kv(cfg, lengths, int(lengths.max()), tag="bench.ctx")
    cache.set_context(Kc, Vc, lengths)
    ws = dfl.Workspace(model, B, gamma)
    len0 = torch.as_tensor(np.asarray(lengths, dtype=np.int32), device="cuda")
    feat = dfl.to_device(gen.features(cfg, B, gamma, tag="bench.if.feat"), "cuda")
    n_rows = 6                                   # about the planted mean accept length
    n_new = torch.full((B,), n_rows, dtype=torch.int32, device="cuda")
    anchor = torch.as_tensor(gen.tokens(cfg, "bench.if.anchor", (B,)), device="cuda")
    draft = torch.zeros((B, gamma - 1), dtype=torch.int32, device="cuda")

    def timed(inject):
        def step():
            cache.len.copy_(len0)
            inject(model, cache, feat, n_new, ws)
            dfl.draft_block(model, cache, gamma, anchor, draft, ws)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        return e0.elapsed_time(e1) * 1000.0 / args.steps

    us_kv = timed(dfl.inject_kv)
    us_if = timed(dfl.inject_kv_input_fusion)
    print(json.dumps({"metric": "conditioning + drafting time, input fusion vs KV injection", "value": round(us_if, 1),
                      "unit": "us", "higher_is_better": False, "steps": args.steps, "warmup": args.warmup,
                      "dtype": cfg.dtype, "kv_injection_us": round(us_kv, 1), "input_fusion_us": round(us_if, 1),
                      "ratio": round(us_if / us_kv, 3), "new_context_rows": n_rows,
                      "config": {"workload": f"{cfg.name}: {SHAPES.get(cfg.name, cfg.name)}, batch {B}, gamma {gamma}, "
                                             f"context {int(lengths.mean())}", "batch": B, "gamma": gamma}}),
          flush=True)


def target_verify(args, dfl, cfg, gen, torch):
    """The verifying target's forward over one block: a Qwen3-8B-shaped target (the drafter's
    layer recipe, 36 layers, untied LM head) checks anchor + gamma-1 drafts at context C, keeping
    the block's K/V rows, tapping 5 evenly spread layers' hidden states for the drafter and taking
    every row's argmax.  HBM-bound at small batch: every weight once plus the context K/V."""
    import numpy as np
    B, gamma, C = args.batch, cfg.gamma, cfg.ctx
    L = 36
    tcfg = cfg.with_(n_layers=L, batch=B, index=cfg.index + 1000)
    cap = (C + 2 * cfg.gamma_max + 63) // 64 * 64
    t0 = time.time()
    W = gen.weights(tcfg)
    W["w_fuse"] = None
    log(f"target weights generated {time.time() - t0:.1f}s")
    model = dfl.Model(tcfg, W, device="cuda", max_batch=B, kv_capacity=cap)
    del W
    cache = dfl.Cache(model)
    lengths = np.full(B, C, dtype=np.int32)
    Kc, Vc = gen.context_kv(tcfg, lengths, C, tag="bench.target.ctx")
    cache.set_context(Kc, Vc, lengths)
    del Kc, Vc
    ws = dfl.Workspace(model, B, 0)
    taps = [int(round(t)) for t in np.linspace(1, L, cfg.n_feat)]
    log(f"target uploaded {time.time() - t0:.1f}s; taps {taps}; workspace {ws.nbytes / 2**20:.1f} MiB")
    NT = 8
    toks = [torch.as_tensor(gen.tokens(tcfg, f"bench.target.tok.{i}", (B, gamma)).astype(np.int32), device="cuda")
            for i in range(NT)]
    y = torch.empty((B, gamma), dtype=torch.int32, device="cuda")
    feat = torch.empty((B, gamma, len(taps), cfg.hidden), dtype=model.storage_dtype, device="cuda")
    len_base = torch.as_tensor(lengths, device="cuda")

    def step(i):
        cache.len[:B].copy_(len_base)
        dfl.target_forward(model, cache, toks[i % NT], y, ws, feat=feat, taps=taps)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    times = []
    for r in range(args.reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / args.steps)
    assert int(cache.status.item()) == 0
    ms = statistics.median(times)
    e = tcfg.elem_bytes
    H, D = cfg.hidden, cfg.head_dim
    w_bytes = L * ((cfg.n_q + 2 * cfg.n_kv) * D * H + cfg.n_q * D * H + 3 * cfg.inter * H) * e + cfg.vocab * H * e
    kv_bytes = L * B * cfg.n_kv * C * D * 2 * e
    io_bytes = B * gamma * (L * 2 * cfg.n_kv * D + len(taps) * H) * e
    total = w_bytes + kv_bytes + io_bytes
    gbs = total / (ms * 1e-3) / 1e9
    log(f"target forward {ms * 1000:.1f} us ({gbs:.0f} GB/s of {total / 1e9:.2f} GB), reps "
        f"{[round(t * 1000, 1) for t in times]}")
    print(json.dumps({"metric": "target verification forward time", "value": round(ms * 1000, 1), "unit": "us",
                      "higher_is_better": False, "steps": args.steps, "warmup": args.warmup, "dtype": cfg.dtype,
                      "data": "synthetic (seeded random-init target weights and context K/V)",
                      "config": {"workload": f"Qwen3-8B-shaped target ({L} layers, hidden {H}, GQA "
                                             f"{cfg.n_q}/{cfg.n_kv}, vocab {cfg.vocab}), batch {B}, block of "
                                             f"{gamma} rows at context {C}, {len(taps)} tapped layers {taps}",
                                 "batch": B, "gamma": gamma, "context": C, "layers": L},
                      "verified_rows_per_s": round(B * gamma / (ms * 1e-3), 1),
                      "roofline": {"bound": "hbm", "kernel": "whole forward", "achieved": round(gbs, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "algorithmic_bytes": int(total)}}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C3")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="per thread setting")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probes", action="store_true",
                    help="also run the HBM-read and MFMA ceiling probes (libdflash_probe.so)")
    ap.add_argument("--trace-cycles", type=int, default=20)
    ap.add_argument("--gamma", type=int, default=0, help="block size (default: the configuration's)")
    ap.add_argument("--layers", type=int, default=0, help="draft layers (default: the configuration's)")
    ap.add_argument("--prefill", action="store_true",
                    help="time the injection of a whole context's feature rows instead of the cycle")
    ap.add_argument("--target", action="store_true",
                    help="time the verifying target's forward over one block (36-layer target of the config's shape)")
    ap.add_argument("--input-fusion", action="store_true",
                    help="time input-fusion conditioning + drafting beside KV injection + drafting")
    ap.add_argument("--loss", action="store_true",
                    help="time the drafter's position-weighted block cross-entropy beside the drafting pass")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 5 times (a plain copy kernel of known size, "
                         "to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_diffusion_drafter_states_amd as dfl
    from block_diffusion_drafter_states_amd import _abi
    import synth
    from synth import gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 5 x {n} bytes read and written")
        return
    dfl.lib()

    cfg = synth.get_config(args.config)
    if args.gamma:
        cfg = cfg.with_(gamma=args.gamma, gammas=None)
    if args.layers:
        cfg = cfg.with_(n_layers=args.layers)
    if args.prefill:
        prefill(args, dfl, cfg, gen, torch)
        return
    if args.target:
        target_verify(args, dfl, cfg, gen, torch)
        return
    if args.loss:
        block_loss_leg(args, dfl, cfg, gen, torch)
        return
    if args.input_fusion:
        input_fusion_leg(args, dfl, cfg, gen, torch)
        return
    B = args.batch
    cfg = cfg.with_(batch=B)
    gamma = cfg.gamma_max
    # block size of cycle i (a configuration with several block sizes cycles through them)
    gseq = list(cfg.gammas) if cfg.gammas else [cfg.gamma]
    gam = lambda i: gseq[i % len(gseq)]
    lengths = gen.context_lengths(cfg)
    cap = (int(lengths.max()) + 2 * cfg.gamma_max + 63) // 64 * 64
    dev = "cuda"
    K_steps, W_steps = args.steps, args.warmup

    t0 = time.time()
    W = gen.weights(cfg)
    log(f"weights generated {time.time() - t0:.1f}s")
    model = dfl.Model(cfg, W, device=dev, max_batch=B, kv_capacity=cap)
    cache = dfl.Cache(model)
    Kc, Vc = gen.context_kv(cfg, lengths, int(lengths.max()), tag="bench.ctx")
    cache.set_context(Kc, Vc, lengths)
    ws = dfl.Workspace(model, B, gamma)
    log(f"uploaded {time.time() - t0:.1f}s; workspace {ws.nbytes / 2**20:.1f} MiB, cap {cap}")

    NP = 8
    feats_host = [gen.features(cfg, B, gamma, tag=f"bench.feat.{i}") for i in range(NP)]
    feats = [dfl.to_device(f, dev) for f in feats_host]
    plant_k = [gen.planted_accept(cfg, (B,), gam(i), tag=f"bench.k.{i}") for i in range(K_steps)]
    anchor0 = gen.anchors(cfg, B, tag="bench.anchor")
    len_base = torch.as_tensor(lengths, dtype=torch.int32, device=dev)
    # the context length is held at the configured value every cycle (the cycle's injection
    # advances it): one fill kernel when every sequence has the same length, else a copy
    same_len = int(lengths[0]) if len(set(int(x) for x in lengths)) == 1 else None

    def hold_len():
        if same_len is not None:
            cache.len[:B].fill_(same_len)
        else:
            cache.len[:B].copy_(len_base)
    acc = torch.zeros((K_steps + 1, B), dtype=torch.int32, device=dev)      # accept_len per cycle
    nxt = torch.zeros((K_steps + 1, B), dtype=torch.int32, device=dev)      # next anchor per cycle
    drafts = [torch.zeros((B, gam(i) - 1), dtype=torch.int32, device=dev) for i in range(K_steps)]
    ytgt = [torch.zeros((B, gam(i)), dtype=torch.int32, device=dev) for i in range(K_steps)]
    committed = {g: torch.zeros((B, g), dtype=torch.int32, device=dev) for g in gseq}
    tau0 = torch.as_tensor(plant_k[-1] + 1, dtype=torch.int32, device=dev)

    def reset():
        acc[0].copy_(tau0)
        nxt[0].copy_(torch.as_tensor(anchor0, device=dev))

    def cycle(i, trace=None):
        hold_len()
        g = gam(i)
        if trace is None:
            dfl.inject_kv(model, cache, feats[i % NP], acc[i], ws)
            dfl.draft_block(model, cache, g, nxt[i], drafts[i], ws)
        else:
            _abi.check(dfl.lib().dflash_inject_kv_traced(
                ctypes.byref(model.c), ctypes.byref(model.w), ctypes.byref(cache.s), B, feats[i % NP].data_ptr(),
                gamma, acc[i].data_ptr(), ws.ptr(), ws.nbytes, dfl._stream_ptr(None), ctypes.byref(trace[0])),
                "inject_traced")
            _abi.check(dfl.lib().dflash_draft_block_traced(
                ctypes.byref(model.c), ctypes.byref(model.w), ctypes.byref(cache.s), B, g, nxt[i].data_ptr(),
                drafts[i].data_ptr(), None, None, ws.ptr(), ws.nbytes, dfl._stream_ptr(None),
                ctypes.byref(trace[1])), "draft_traced")
        dfl.verify(drafts[i], ytgt[i], acc[i + 1], committed[g], nxt[i + 1])

    # ---- planning pass (untimed): record drafts, plant target tokens
    t1 = time.time()
    reset()
    for i in range(K_steps):
        hold_len()
        dfl.inject_kv(model, cache, feats[i % NP], acc[i], ws)
        dfl.draft_block(model, cache, gam(i), nxt[i], drafts[i], ws)
        d = drafts[i].cpu().numpy()
        ytgt[i].copy_(torch.as_tensor(gen.planted_targets(cfg, d, plant_k[i], tag=f"bench.y.{i}")))
        dfl.verify(drafts[i], ytgt[i], acc[i + 1], committed[gam(i)], nxt[i + 1])
    torch.cuda.synchronize()
    status = int(cache.status.item())
    assert status == 0, f"device status {status}"
    log(f"planning pass {time.time() - t1:.1f}s")

    # ---- warm-up + timed repetitions
    reset()
    for i in range(min(W_steps, K_steps)):
        cycle(i)
    torch.cuda.synchronize()
    times = []
    for r in range(args.reps):
        reset()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K_steps):
            cycle(i)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
        taus = acc[1:].cpu().numpy()
        want = np.stack(plant_k) + 1
        assert np.array_equal(taus, want), "timed pass did not reproduce the planted accept lengths"
    ms_total = statistics.median(times)
    ms_per = ms_total / K_steps
    cps = 1000.0 / ms_per
    tau_mean = float(np.mean(np.stack(plant_k) + 1))
    log(f"cycles: {ms_per * 1000:.1f} us/cycle ({cps:.1f} cycles/s), reps {[round(t / K_steps * 1000, 1) for t in times]}")

    # ---- per-launch timing with library-recorded events
    hip = Hip()
    CAP = 256
    names_arr = [(ctypes.c_char_p * CAP)(), (ctypes.c_char_p * CAP)()]
    probe = [_abi.dflash_trace(events=None, capacity=CAP, count=0,
                               names=ctypes.cast(names_arr[k], ctypes.POINTER(ctypes.c_char_p))) for k in range(2)]
    reset()
    cycle(0, trace=probe)
    torch.cuda.synchronize()
    names = [[names_arr[k][i].decode() for i in range(probe[k].count)] for k in range(2)]
    NT = min(args.trace_cycles, K_steps)
    per_cycle = []
    for i in range(NT):
        tr = []
        for k in range(2):
            n = probe[k].count
            evs = (ctypes.c_void_p * (2 * n))(*[hip.event() for _ in range(2 * n)])
            t = _abi.dflash_trace(events=ctypes.cast(evs, ctypes.POINTER(ctypes.c_void_p)), capacity=n, count=0,
                                  names=None)
            t._evs = evs
            tr.append(t)
        per_cycle.append(tr)
    reset()
    for i in range(NT):
        cycle(i, trace=per_cycle[i])
    torch.cuda.synchronize()
    kern = {}
    for i in range(NT):
        for k in range(2):
            evs = per_cycle[i][k]._evs
            for j, nm in enumerate(names[k]):
                kern.setdefault(nm, []).append(hip.elapsed_ms(evs[2 * j], evs[2 * j + 1]))
            for e in evs:
                hip.destroy(e)
    kern_us = {nm: round(1000.0 * sum(v) / NT, 2) for nm, v in kern.items()}     # per cycle (all launches)
    lm = kern["lm_head_argmax"]
    lm_avg_ms = sum(lm) / len(lm)
    g_mean = float(np.mean([gam(i) for i in range(K_steps)]))
    lm_bytes = int(cfg.vocab * cfg.hidden * cfg.elem_bytes + B * g_mean * cfg.hidden * cfg.elem_bytes)  # W_lm + rows
    lm_gbs = lm_bytes / (lm_avg_ms * 1e-3) / 1e9
    log(f"lm_head_argmax {lm_avg_ms * 1000:.1f} us -> {lm_gbs:.0f} GB/s; per-cycle kernel us {kern_us}")

    parts, bytes_cycle = algorithmic_bytes(cfg, B, float(np.mean(lengths)), tau_mean)
    cycle_frac = bytes_cycle * cps / (HBM_PEAK_GBS * 1e9)
    result = {
        "metric": METRIC,
        "value": round(cps, 2),
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": round(ms_per, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded random-init drafter weights, N(0,1) target features and context K/V, "
                "planted target tokens)",
        "config": {"workload": f"{cfg.name}: {SHAPES.get(cfg.name, cfg.name)}, {cfg.n_layers} layers, batch {B}, "
                               f"gamma {'/'.join(str(g) for g in gseq)}, context {int(lengths.mean())}",
                   "batch": B, "gamma": gseq[0] if len(gseq) == 1 else gseq, "context": int(lengths.mean()),
                   "hidden": cfg.hidden, "layers": cfg.n_layers, "vocab": cfg.vocab, "parallelism": "single GPU"},
        "draft_tokens_per_s": round(cps * B * (g_mean - 1), 1),
        "committed_tokens_per_s": round(cps * B * tau_mean, 1),
        "planted_mean_accept_len": round(tau_mean, 3),
        "bytes_per_cycle": int(bytes_cycle),
        "hbm_roofline_frac": round(cycle_frac, 4),
        # the dominant kernel (the measurement contract's `roofline`); the whole cycle's fraction
        # is repeated inside it and in `cycle_roofline`, so no reader takes one for the other
        "roofline": {"bound": "hbm", "kernel": "lm_head_argmax (dominant kernel, not the whole cycle)",
                     "achieved": round(lm_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name == "qwen3_8b_drafter" and B == 1),
                     "traffic_unit": "bytes/launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes_per_launch": lm_bytes,
                     "avg_launch_us": round(lm_avg_ms * 1000, 2),
                     "whole_cycle_frac": round(cycle_frac, 4)},
        "cycle_roofline": {"bound": "hbm", "kernel": "whole cycle", "achieved": round(bytes_cycle * cps / 1e9, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(cycle_frac, 4),
                           "algorithmic_bytes_per_cycle": int(bytes_cycle)},
        # per-launch times from events the library records around every launch of separate
        # traced cycles: the events themselves add time, so these sum to more than ms_per_step
        "kernels_us_per_cycle_event_bracketed": kern_us,
        "kernels_us_per_cycle_sum": round(sum(kern_us.values()), 1),
    }
    peaks = None
    if args.probes:
        # plain probe kernels on the same GPU: a grid-stride read (a floor for the attainable read
        # rate: the LM head's direct-to-LDS stream is faster) and independent-MFMA loops
        peaks = measured_peaks(torch)
        result["probes"] = peaks
    if B > 1:
        # contraction throughput (the dense-MFMA regime of large batches): the cycle's GEMM flops
        # over the whole cycle and over the projection launches alone
        gf = gemm_flops(cfg, B, g_mean, tau_mean)
        gemm_us = sum(v for k, v in kern_us.items() if k in GEMM_LAUNCHES)
        peak = MFMA_PEAK_TFLOPS[cfg.dtype]
        result["mfma"] = {"gemm_gflop_per_cycle": round(gf / 1e9, 1), "peak_tflops": peak,
                          "frac_whole_cycle": round(gf * cps / 1e12 / peak, 4),
                          "frac_gemm_launches": round(gf / (gemm_us * 1e-6) / 1e12 / peak, 4),
                          "gemm_us_per_cycle": round(gemm_us, 1)}
        if peaks:
            result["mfma"]["frac_gemm_launches_of_mfma_probe"] = round(
                gf / (gemm_us * 1e-6) / 1e12 / peaks["mfma_bf16_TFLOPs"], 4)
    if not args.no_cpu_baseline:
        Kh, Vh = gen.context_kv(cfg, lengths, cap, tag="bench.ctx")
        result["cpu_baseline"] = cpu_oracle_baseline(cfg, W, Kh, Vh, lengths, feats_host, anchor0, plant_k, gseq,
                                                     args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
