"""Benchmark of the Simple GLA mixer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only PART]

Prints ONE JSON line.  The headline `value` is chunked-prefill throughput
(tokens/s) on the training-shape workload: B=8, H=16, T=2048 (16 chunks of
128), dk=96, dv=192, bf16 q/k/v, fp32 log-decay, state and accumulation,
bf16 output.  One step = one gla_chunk_fwd call over that batch, inputs
resident in HBM.  The same line carries, measured in the same run:
  decode    batched decode step, 1,280 sequences x 24 layers x 64 steps,
            fp32 state read and written in place (GB/s of state traffic)
  backward  chunked backward, B=4, H=16, T=4096 (tokens/s), and on fp32
            inputs and outputs at B=1, T=2048 (backward.fp32)
  long_context  prefill B=1, T=65536 with a non-zero initial state
  packed    serving prefill: 16 prompts of 2,048-8,192 tokens packed along
            one token axis, final states written into a 1,280-slot pool
  fused     the headline prefill reading q, k, v in place from the fused
            [8, 2048, 9216] projection output (strided views, no copies),
            and the same with the output gate o * SiLU(gate) fused in
  conv      causal depth-wise conv1d (width 4) + SiLU ahead of the mixer,
            B=8, T=2048, D=3,072, bf16 in/out, window of the last four inputs kept
            per sequence (float32)
  fp32      prefill B=1, T=2048 with fp32 inputs and outputs
  roofline  the prefill walk kernel against the HBM roof (HIP events)
  mfma_util the prefill's MFMA utilisation beside its ceiling (what the HBM
            roof allows for its FLOPs and bytes) and a vendor-BLAS bf16 GEMM
  prefill_mall_warm  the prefill right after kernels that wrote its inputs
            (part may sit in the memory-side cache); labelled, not headline
  hbm_copy_reference  a plain device copy on rotating buffers: the streaming
            rate this GPU reaches, and each HBM-bound part as a fraction of it
  device    the GPU's properties and the rates of a plain read, write and
            fp32 GEMM it reaches (reference points)
  decode_after_prefix  the decode step on 1,280-slot pools whose states
            came from 2,048- and from 8,192-token prefills: equal times
  cpu_baseline  the fp64 oracle on the host cores, whole workload
  cpu_baseline_decode  the oracle's decode step over one layer's 1,280 x 16
            slots for 4 steps, extrapolated to 24 layers (labelled)
  parity    sampled max|err|/rms(ref) against the oracle for this run

--only PART runs a single part a few times (for profiler counter passes):
prefill | decode | backward | packed | conv | fused | long | copy (a plain
1 GiB device copy used to scale the HBM byte counters).
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

import numpy as np  # noqa: E402

import gen  # noqa: E402

METRIC = "GLA prefill tokens/s + MFMA util; decode state-update GB/s (H16 dk96 dv192)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
F32_MFMA_PEAK_TFLOPS = 157.3
H, DK, DV, CH = 16, 96, 192, 128

# Algorithmic work per token-head (dense 128-token chunks):
#   forward  = 2*C*dk + 2*C*dv + 2*dk*dv + 2*dk*dv = 147,456 flop
#   backward = 2*C*(3dk + 2dv) + 3*2*dk*dv   chunk gradients
#            + 2*dk*dv                        forward states recomputed
#            + 2*dk*dv                        reverse state gradient
#            = 356,352 flop
FWD_FLOP_PER_TH = 2 * CH * DK + 2 * CH * DV + 4 * DK * DV
BWD_FLOP_PER_TH = 2 * CH * (3 * DK + 2 * DV) + 10 * DK * DV


def mfma_ceiling(flops, nbytes, peak_tflops, hbm_gbs=HBM_PEAK_GBS):
    """The highest MFMA utilisation the roofline allows: the time the FLOPs
    take at peak over the time the algorithmic bytes take at the HBM peak,
    capped at 1 (a part whose bytes take longer can reach only that share)."""
    t_flop = flops / (peak_tflops * 1e12)
    t_byte = nbytes / (hbm_gbs * 1e9)
    return 1.0 if t_byte <= t_flop else t_flop / t_byte


def fwd_bytes(B, T, in_b, out_b, s0=False):
    """q, k, v read, g read, o written once; S_T written (and S0 read)."""
    th = B * T * H
    per = (2 * DK + DV) * in_b + 4 + DV * out_b
    return th * per + B * H * DK * DV * 4 * (2 if s0 else 1)


def packed_bytes(n_tokens, n_seq, in_b, out_b, init=False):
    """Packed prefill: every token's q, k, v, g read and o written once; each
    sequence's final state written to its slot (and its initial one read)."""
    per = (2 * DK + DV) * in_b + 4 + DV * out_b
    return n_tokens * H * per + n_seq * H * DK * DV * 4 * (2 if init else 1)


def bwd_bytes(B, T, in_b, out_b):
    th = B * T * H
    return th * ((2 * DK + 2 * DV) * in_b + 4 + (2 * DK + DV) * out_b + 4)


def decode_bytes(n_seq, in_b=2, out_b=4, q16=False):
    """Algorithmic bytes of one decode step: the state read and written (fp32,
    or int16 mantissas plus an int32 exponent per column), q, k, v, g and o."""
    state = DK * DV * 2 + DV * 4 if q16 else DK * DV * 4
    per = 2 * state + (2 * DK + DV) * in_b + 4 + DV * out_b
    return n_seq * H * per


# --------------------------------------------------------------------------
# CPU baseline: the oracle, unchanged, over independent (b, h) pairs
# --------------------------------------------------------------------------

_CPU_INPUTS = {}


def _oracle_pair(args):
    b, h = args
    import oracle
    d = _CPU_INPUTS                      # inherited from the parent through fork
    sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
    t0 = time.perf_counter()
    oracle.forward(d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl], None)
    return time.perf_counter() - t0


def cpu_baseline(max_pairs=128, seed=0, min_cpu_s=10.0, max_passes=6):
    """Time the oracle on the prefill workload, one process per core.  The
    whole workload is a few seconds of CPU work, so it is walked in whole
    passes until at least min_cpu_s of CPU work has been timed."""
    import multiprocessing as mp
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores = min(len(os.sched_getaffinity(0)), 16)
    B = gen.WORKLOADS["fwd_bf16_b8_t2048"]["B"]
    pairs = [(b, h) for b in range(B) for h in range(H)][:max_pairs]
    _CPU_INPUTS.clear()
    _CPU_INPUTS.update(gen.make_inputs("fwd_bf16_b8_t2048", seed=seed))
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    os.environ["MKL_NUM_THREADS"] = "1"
    ctx = mp.get_context("fork")
    per, passes = [], 0
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        while passes < max_passes and (passes == 0 or sum(per) < min_cpu_s):
            if threadpool_limits is not None:
                with threadpool_limits(1):
                    per += pool.map(_oracle_pair, pairs, chunksize=1)
            else:
                per += pool.map(_oracle_pair, pairs, chunksize=1)
            passes += 1
    wall = time.perf_counter() - t0
    T = gen.WORKLOADS["fwd_bf16_b8_t2048"]["T"]
    tokens = passes * len(pairs) / H * T * 1.0
    return {"value": tokens / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": (f"fp64 token-by-token oracle over {len(pairs)} of the {B * H} (b,h) "
                       f"sequences of the B={B} T={T} prefill workload, {passes} passes, one process "
                       f"per core (1 BLAS thread each); {sum(per):.1f} s of CPU work, {wall:.2f} s wall"),
            "cpu_seconds": sum(per)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_decode_chunk(args):
    """`steps` oracle decode steps over `n` slots of one layer; returns the
    CPU seconds of the steps alone (input generation is not timed)."""
    chunk, n, steps = args
    import oracle
    S = gen.make_decode_state(n, seed=1000 + chunk)
    spent = 0.0
    for s in range(steps):
        x = gen.make_decode_step(n, s, seed=1000 + chunk)
        t0 = time.perf_counter()
        _, S = oracle.step(S, x["q"], x["k"], x["v"], x["g"])
        spent += time.perf_counter() - t0
    return spent


def cpu_decode_baseline(n_seq=1280, per_task=80, steps=4, layers=24, total_steps=64):
    """The oracle's decode step over every slot of one layer (n_seq x 16 heads)
    for `steps` steps, one process per core; the 24-layer, 64-step figure is a
    linear extrapolation of that and is labelled as one.  The full fp64 state
    of 24 layers (some 72 GB) is never held."""
    import multiprocessing as mp
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores = min(len(os.sched_getaffinity(0)), 16)
    tasks = [(c, per_task, steps) for c in range(n_seq // per_task)]
    os.environ["OMP_NUM_THREADS"] = "1"
    with mp.get_context("fork").Pool(cores) as pool:
        if threadpool_limits is not None:
            with threadpool_limits(1):
                per = pool.map(_oracle_decode_chunk, tasks, chunksize=1)
        else:
            per = pool.map(_oracle_decode_chunk, tasks, chunksize=1)
    cpu_s = sum(per)
    used = min(cores, len(tasks))
    us_layer_step = cpu_s / used / steps * 1e6       # the steps' CPU time shared over the cores used
    return {"us_per_layer_step": us_layer_step,
            "tokens_per_s_24_layers": n_seq / (layers * us_layer_step * 1e-6),
            "cores": used, "kind": "oracle", "extrapolated": True,
            "sample": (f"fp64 oracle decode step over all {n_seq} x 16 slots of one layer for {steps} steps "
                       f"({len(tasks)} tasks of {per_task} sequences, one process per core); per layer-step "
                       f"time = {cpu_s:.1f} CPU s of the steps / {used} cores / {steps}; tokens/s for "
                       f"{layers} layers x {total_steps} steps extrapolated linearly from it")}


# --------------------------------------------------------------------------
# GPU parts
# --------------------------------------------------------------------------

def _gpu():
    import torch
    import linear_attention_sequence_simple_amd as gla
    gla.lib()
    return torch, gla


def _dev_inputs(torch, d, in_dtype):
    dev = torch.device("cuda", 0)
    T = lambda x, dt: None if x is None else torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(dt)
    return (T(d["q"], in_dtype), T(d["k"], in_dtype), T(d["v"], in_dtype), T(d["g"], torch.float32),
            T(d["S0"], torch.float32), T(d.get("dO"), in_dtype))


def _time_calls(torch, fn, steps, warmup, warm_ms=0.0):
    """Mean device time per call of fn(): HIP events on the current stream
    bracket the `steps` timed calls, which run back to back.

    The GPU's clocks take some 50 ms of sustained load to reach their steady
    level from idle: `warmup` untimed calls run first, then more untimed calls
    until at least warm_ms of warm-up have passed (the first part measured
    asks for 100 ms, the parts measured after the host has prepared their
    inputs for 30 ms).  A short spin of the device (about 0.4 ms)
    is queued ahead of the timed region so that the binding's host-side
    marshalling (some 14 us per call, below every kernel's duration) never
    leaves the device idle; a longer spin lets the clocks drop again.  The
    events sit outside the calls, so nothing is inserted between the kernels
    being timed.  Returns (ms per call, wall seconds)."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(1e6))
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def _bf16_out_ratio(got, ref, tol):
    """Largest |got - ref| / (tol rms(ref) + 2^-8 |ref|): the elementwise bound
    for outputs rounded to bf16 (at most 1 passes).  2^-8 |ref| is bf16's half
    ulp at the bottom of a binade, so rounding alone can bring this close to 1."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = tol * math.sqrt(float(np.mean(ref * ref))) + 2.0 ** -8 * np.abs(ref)
    return float(np.max(np.abs(got - ref) / bound))


def _rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / math.sqrt(float(np.mean(ref * ref))))


def bench_prefill(torch, gla, steps, warmup, parity=True, sets=3):
    """The headline: one gla_chunk_fwd call per step on the training shape,
    bf16 in and out.  The calls cycle over `sets` input/output sets (seeds
    0..sets-1; 907 MB in all, more than the 256 MB memory-side cache), so
    every call reads its inputs from HBM.  Parity reads the timed calls' own
    bf16 o of set 0 on sampled (b, h) pairs, and also checks an fp32-output
    call on the same inputs."""
    ds = [gen.make_inputs("fwd_bf16_b8_t2048", seed=s) for s in range(sets)]
    d = ds[0]
    B, T = d["meta"]["B"], d["meta"]["T"]
    ins = [_dev_inputs(torch, x, torch.bfloat16)[:4] for x in ds]
    dev = ins[0][0].device
    outs = [(torch.empty((B, T, H, DV), dtype=torch.bfloat16, device=dev),
             torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)) for _ in range(sets)]
    dims = gla.GlaDims(B, T, H, DK, DV, CH, gla.GLA_BF16, gla.GLA_BF16)
    ws_bytes = gla.gla_workspace_size(gla.GLA_OP_FWD, dims)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    it = [0]

    def fn():
        i = it[0] % sets
        it[0] += 1
        q, k, v, g = ins[i]
        gla.gla_chunk_fwd(q, k, v, g, None, out_dtype=torch.bfloat16, o=outs[i][0], S_T=outs[i][1], workspace=ws)
    ms, wall = _time_calls(torch, fn, steps, warmup, warm_ms=100)
    tokens = B * T
    nbytes = fwd_bytes(B, T, 2, 2)
    flops = FWD_FLOP_PER_TH * B * T * H
    res = {"ms": ms, "tokens_per_s": tokens / (ms * 1e-3), "bytes": nbytes,
           "flops": flops, "GBps": nbytes / (ms * 1e-3) / 1e9,
           "mfma_util": flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
           "mfma_ceiling": mfma_ceiling(flops, nbytes, BF16_PEAK_TFLOPS), "launches": 1 if ws_bytes == 0 else 3,
           "input_sets": sets, "wall_s": wall}
    if parity:
        import oracle
        torch.cuda.synchronize()
        q, k, v, g = ins[0]
        o_timed = outs[0][0].float().cpu().numpy()
        S_timed = outs[0][1].cpu().numpy()
        o32, _ = gla.gla_chunk_fwd(q, k, v, g, None, out_dtype=torch.float32, want_state=False)
        torch.cuda.synchronize()
        bs, hs = [0, 4, 7], [0, 8, 15]
        sub = lambda x: x[np.ix_(bs, range(T), hs)]
        o_ref, S_ref = oracle.forward(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["g"]), None)
        res["parity"] = {"o_bf16_timed_call_over_bound": _bf16_out_ratio(sub(o_timed), o_ref, 1e-2),
                         "S_T_timed_call": _rel_err(S_timed[np.ix_(bs, hs)], S_ref),
                         "o_fp32_out": _rel_err(o32.cpu().numpy()[np.ix_(bs, range(T), hs)], o_ref),
                         "sample": "(b,h) in {0,4,7}x{0,8,15}, all 2048 tokens, input set 0; bf16 o of the timed "
                                   "calls against the elementwise bound 1e-2 rms + 2^-8 |ref| (at most 1 passes)"}
    return res


def _per_launch_ms(torch, producer, fn, steps, warm_iters=20):
    """Mean device time of fn() alone when each call follows producer():
    events recorded between the two bracket fn's kernels only (the stream
    runs in order, so the start event completes once the producer's kernels
    have)."""
    for _ in range(warm_iters):
        producer()
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda._sleep(int(1e6))
    for a, b in ev:
        producer()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps


def bench_prefill_mall_warm(torch, gla, steps):
    """The headline prefill with its inputs just written by a preceding
    kernel, as the projection that produces q, k, v and the log-decay would
    leave them: part of them may still sit in the memory-side (MALL) cache.
    Beside it the same call after a producer that writes as many bytes to
    other buffers, so both follow the same preceding work.  Reported apart
    from the headline figure, which reads inputs that are resident in HBM."""
    d = gen.make_inputs("fwd_bf16_b8_t2048", seed=0)
    B, T = d["meta"]["B"], d["meta"]["T"]
    q, k, v, g, _, _ = _dev_inputs(torch, d, torch.bfloat16)
    src = [x.clone() for x in (q, k, v, g)]
    other = [torch.empty_like(x) for x in (q, k, v, g)]
    o = torch.empty((B, T, H, DV), dtype=torch.bfloat16, device=q.device)
    S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device=q.device)
    fn = lambda: gla.gla_chunk_fwd(q, k, v, g, None, out_dtype=torch.bfloat16, o=o, S_T=S_T)

    def write_inputs():
        for dst, x in zip((q, k, v, g), src):
            dst.copy_(x)

    def write_other():
        for dst, x in zip(other, src):
            dst.copy_(x)

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=q.device)

    def write_flush():
        flush.zero_()

    warm = _per_launch_ms(torch, write_inputs, fn, steps)
    cold = _per_launch_ms(torch, write_other, fn, steps)
    flushed = _per_launch_ms(torch, write_flush, fn, steps)
    del flush
    nbytes = fwd_bytes(B, T, 2, 2)
    in_bytes = sum(x.numel() * x.element_size() for x in src)
    return {"label": "MALL-warm: inputs written by the kernels just before the call (not the headline figure)",
            "ms_inputs_just_written": warm, "ms_after_other_writes": cold,
            "tokens_per_s_inputs_just_written": B * T / (warm * 1e-3),
            "tokens_per_s_after_other_writes": B * T / (cold * 1e-3),
            "speedup": cold / warm, "input_bytes_written_before_each_call": in_bytes,
            "ms_cold_after_512MB_flush": flushed,
            "tokens_per_s_cold_after_512MB_flush": B * T / (flushed * 1e-3),
            "GBps_algorithmic_inputs_just_written": nbytes / (warm * 1e-3) / 1e9,
            "note": "events bracket each gla_chunk_fwd launch alone; the producer is four torch copies "
                    "into the call's q, k, v, g (or, beside it, into other buffers of the same sizes); "
                    "the cold figure follows a 512 MB fill of another buffer, twice the memory-side cache"}


def bench_decode_after_prefix(torch, gla, steps=32, n=1280, group=160, piece=2048):
    """Decode step time on pools whose states were built by prefills over
    2,048 and over 8,192 tokens.  Each pool's n slots are filled `group`
    sequences at a time by chained prefills of `piece` tokens (the final
    state of one piece is the initial state of the next), the last writing
    into the slots; every piece gets fresh inputs.  The state has the same
    size whatever the prefix, so the two times must agree.  These prefill
    inputs feed no parity check: they are drawn on the device from a seeded
    torch generator (N(0,1)/sqrt(96) for q, k, v in bf16, logsigmoid(N(0,1) + 4)
    for the log-decay)."""
    dev = torch.device("cuda", 0)
    gen_t = torch.Generator(device=dev)
    gen_t.manual_seed(6)
    rnd = lambda *shape: torch.randn(shape, generator=gen_t, device=dev)
    sc = 1.0 / math.sqrt(DK)
    q = torch.empty((group, piece, H, DK), dtype=torch.bfloat16, device=dev)
    k, v = torch.empty_like(q), torch.empty((group, piece, H, DV), dtype=torch.bfloat16, device=dev)
    g = torch.empty((group, piece, H), dtype=torch.float32, device=dev)

    def draw():
        q.copy_(rnd(group, piece, H, DK) * sc)
        k.copy_(rnd(group, piece, H, DK) * sc)
        v.copy_(rnd(group, piece, H, DV) * sc)
        g.copy_(torch.nn.functional.logsigmoid(rnd(group, piece, H) + 4.0))

    o = torch.empty((group, piece, H, DV), dtype=torch.bfloat16, device=dev)
    tmp = [torch.empty((group, H, DK, DV), dtype=torch.float32, device=dev) for _ in range(2)]
    pools = {}
    for prefix in (2048, 8192):
        pool = gla.gla_state_alloc(n)
        view = pool.view()
        pieces = prefix // piece
        for g0 in range(0, n, group):
            S0 = None
            for r in range(pieces):
                draw()
                dst = view[g0:g0 + group] if r == pieces - 1 else tmp[r % 2]
                gla.gla_chunk_fwd(q, k, v, g, S0, out_dtype=torch.bfloat16, o=o, S_T=dst)
                S0 = dst
        pools[prefix] = pool
    torch.cuda.synchronize()
    a, b = pools[2048].view(), pools[8192].view()
    res = {"state_rms_after_2048_tokens": float(a.pow(2).mean().sqrt()),
           "state_rms_after_8192_tokens": float(b.pow(2).mean().sqrt()),
           "states_max_abs_difference": float((a - b).abs().max())}
    del q, k, v, g, o, tmp
    xs = []
    for st in range(8):
        x = gen.make_decode_step(n, st, seed=2)
        xs.append([torch.from_numpy(x[c]).to(dev).to(torch.bfloat16) for c in ("q", "k", "v")]
                  + [torch.from_numpy(x["g"]).to(dev)])
    out = torch.empty((n, H, DV), dtype=torch.float32, device=dev)
    for prefix, pool in pools.items():
        it = [0]

        def fn():
            x = xs[it[0] % len(xs)]
            it[0] += 1
            gla.gla_recurrent_step(pool, *x, out_dtype=torch.float32, o=out)

        ms, _ = _time_calls(torch, fn, steps, 4, warm_ms=30)
        res[f"us_per_step_after_{prefix}_tokens"] = ms * 1e3
    for pool in pools.values():
        pool.free()
    res["ratio_8192_over_2048"] = res["us_per_step_after_8192_tokens"] / res["us_per_step_after_2048_tokens"]
    res["note"] = (f"{n} sequences x 16 heads, one decode step per call, {steps} timed calls per pool; "
                   "prefix states built by chained bf16 prefills of 2,048 tokens, fresh inputs per piece")
    return res


def device_probe(torch, steps=20):
    """What this GPU reports and reaches: its properties, and the rates of a
    plain 1 GiB read (row sums), write (a fill) and an fp32 GEMM from the vendor
    BLAS.  Reference points beside the nominal peaks, not ceilings."""
    p = torch.cuda.get_device_properties(0)
    n = 1 << 28                                          # 1 GiB of fp32
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    rows = x.view(n // 1024, 1024)
    acc = torch.empty(n // 1024, dtype=torch.float32, device="cuda")
    ms_r, _ = _time_calls(torch, lambda: torch.sum(rows, dim=1, out=acc), steps, 3, warm_ms=30)
    ms_w, _ = _time_calls(torch, lambda: x.fill_(1.0), steps, 3, warm_ms=30)
    del x, rows, acc
    m = 8192
    a = torch.randn((m, m), device="cuda")
    b = torch.randn((m, m), device="cuda")
    c = torch.empty((m, m), device="cuda")
    ms_g, _ = _time_calls(torch, lambda: torch.matmul(a, b, out=c), max(3, steps // 4), 2, warm_ms=30)
    del a, b, c
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "hbm_bytes": p.total_memory, "l2_bytes": getattr(p, "L2_cache_size", None),
            "read_GBps": n * 4 / (ms_r * 1e-3) / 1e9, "write_GBps": n * 4 / (ms_w * 1e-3) / 1e9,
            "fp32_gemm_TFLOPs": 2.0 * m ** 3 / (ms_g * 1e-3) / 1e12,
            "note": "row sums of 1,024 floats over 1 GiB (read; 1 MB written), fill of 1 GiB (write), "
                    "torch.matmul fp32 8192^3; torch's kernels, so lower bounds on what the chip "
                    "reaches; reference points beside the nominal 8 TB/s and 157.3 TFLOP/s"}


def mfma_reference(torch, steps=20):
    """A large bf16 GEMM from the vendor BLAS (through torch.matmul): the dense
    matrix rate this GPU reaches, a reference point beside the nominal peak."""
    n = 8192
    a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    ms, _ = _time_calls(torch, lambda: torch.matmul(a, b, out=c), steps, 3, warm_ms=30)
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    return {"TFLOPs": tf, "frac_of_nominal": tf / BF16_PEAK_TFLOPS,
            "note": f"torch.matmul bf16 {n}x{n}x{n}, {steps} calls; a reference point, not a ceiling"}


def bench_prefill_other(torch, gla, name, in_dtype, out_dtype, steps, warmup):
    d = gen.make_inputs(name, seed=0)
    B, T = d["meta"]["B"], d["meta"]["T"]
    q, k, v, g, S0, _ = _dev_inputs(torch, d, in_dtype)
    dims = gla.GlaDims(B, T, H, DK, DV, CH, gla._dtype_code(in_dtype), gla._dtype_code(out_dtype))
    ws = torch.empty(max(gla.gla_workspace_size(gla.GLA_OP_FWD, dims), 1), dtype=torch.uint8, device=q.device)
    o = torch.empty((B, T, H, DV), dtype=out_dtype, device=q.device)
    S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device=q.device)
    fn = lambda: gla.gla_chunk_fwd(q, k, v, g, S0, out_dtype=out_dtype, o=o, S_T=S_T, workspace=ws)
    ms, _ = _time_calls(torch, fn, steps, warmup, warm_ms=30)
    ib = 2 if in_dtype == torch.bfloat16 else 4
    ob = 2 if out_dtype == torch.bfloat16 else 4
    nbytes = fwd_bytes(B, T, ib, ob, s0=S0 is not None)
    flops = FWD_FLOP_PER_TH * B * T * H
    peak = BF16_PEAK_TFLOPS if in_dtype == torch.bfloat16 else F32_MFMA_PEAK_TFLOPS
    return {"workload": f"prefill B={B} T={T} H=16 {'bf16' if ib == 2 else 'fp32'} in, "
                        f"{'bf16' if ob == 2 else 'fp32'} out" + (", S0 != 0" if S0 is not None else ""),
            "ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "GBps": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_util": flops / (ms * 1e-3) / (peak * 1e12),
            "mfma_ceiling": mfma_ceiling(flops, nbytes, peak),
            "mfma_peak": f"{'bf16' if ib == 2 else 'fp32'} {peak} TFLOP/s"}


def bench_packed(torch, gla, steps, warmup):
    d = gen.make_packed_inputs("serve_prefill_16x2k8k", seed=0, with_pool=False)
    w = d["meta"]
    dev = torch.device("cuda", 0)
    T = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)
    q, k, v = (T(d[n], torch.bfloat16) for n in ("q", "k", "v"))
    g = T(d["g"], torch.float32)
    cu = torch.from_numpy(d["cu_seqlens"]).to(dev)
    slots = torch.from_numpy(d["slot_idx"]).to(dev)
    N, n_seq = int(d["cu_seqlens"][-1]), len(d["slot_idx"])
    pool = gla.gla_state_alloc(w["n_slots"])
    o = torch.empty((N, H, DV), dtype=torch.bfloat16, device=dev)
    dims = gla.GlaDims(n_seq, w["len_hi"], H, DK, DV, CH, gla.GLA_BF16, gla.GLA_BF16)
    ws = torch.empty(max(gla.gla_workspace_size(gla.GLA_OP_FWD, dims), 1), dtype=torch.uint8, device=dev)
    fn = lambda: gla.gla_chunk_fwd_varlen(q, k, v, g, cu, w["len_hi"], pool, slots, init_from_pool=False,
                                          out_dtype=torch.bfloat16, workspace=ws, o=o)
    ms, _ = _time_calls(torch, fn, steps, warmup, warm_ms=30)
    # the same call into a 16-bit pool (final states staged in float32, then encoded)
    pool16 = gla.gla_state_alloc_q16(w["n_slots"])
    ws16 = torch.empty(gla.gla_workspace_size(gla.GLA_OP_FWD_VARLEN_Q16, dims), dtype=torch.uint8, device=dev)
    fn16 = lambda: gla.gla_chunk_fwd_varlen(q, k, v, g, cu, w["len_hi"], pool16, slots, init_from_pool=False,
                                            out_dtype=torch.bfloat16, workspace=ws16, o=o)
    ms16, _ = _time_calls(torch, fn16, steps, 2, warm_ms=30)
    pool16.free()
    del ws16
    fn()                                   # o and the float32 slots of the call checked below
    torch.cuda.synchronize()
    # sampled parity: the longest sequence, head 0, against the oracle (every
    # call starts from zero, so the slot holds that sequence's final state)
    import oracle
    cu_h = d["cu_seqlens"]
    sb = int(np.argmax(np.diff(cu_h)))
    t0, t1 = int(cu_h[sb]), int(cu_h[sb + 1])
    sl = lambda x: x[None, t0:t1, 0:1]
    o_ref, S_ref = oracle.forward(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]))
    got_o = o[t0:t1, 0].float().cpu().numpy()
    got_S = pool.view()[int(d["slot_idx"][sb]), 0].cpu().numpy()
    parity = {"o_bf16_out_over_bound": _bf16_out_ratio(got_o, o_ref[0, :, 0], 1e-2),
              "slot_state": _rel_err(got_S, S_ref[0, 0]),
              "sample": f"sequence {sb} ({t1 - t0} tokens), head 0"}
    pool.free()
    nbytes = packed_bytes(N, n_seq, 2, 2)
    flops = FWD_FLOP_PER_TH * N * H
    lens = w["lengths"]
    return {"workload": f"packed prefill, {n_seq} prompts of {int(lens.min())}-{int(lens.max())} tokens "
                        f"({N} in all), H=16 bf16 in/out, final states into a {w['n_slots']}-slot pool",
            "ms": ms, "tokens_per_s": N / (ms * 1e-3), "GBps": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_util": flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), "bytes": nbytes, "parity": parity,
            "ms_into_16bit_pool": ms16, "tokens_per_s_into_16bit_pool": N / (ms16 * 1e-3)}


def bench_fused(torch, gla, steps, warmup):
    """The headline prefill on views of one [B, T, 9216] buffer holding every
    head's q, k, v and gate per token (blocked by projection), without and
    with the output gate o * SiLU(gate) applied in the walk's epilogue."""
    d = gen.make_inputs("fwd_bf16_b8_t2048", seed=0, with_gate=True)
    B, T = d["meta"]["B"], d["meta"]["T"]
    dev = torch.device("cuda", 0)
    buf = torch.zeros((B, T, H * (2 * DK + 2 * DV)), dtype=torch.bfloat16, device=dev)
    views = (buf[..., :H * DK].unflatten(-1, (H, DK)), buf[..., H * DK:2 * H * DK].unflatten(-1, (H, DK)),
             buf[..., 2 * H * DK:2 * H * DK + H * DV].unflatten(-1, (H, DV)))
    gate = buf[..., 2 * H * DK + H * DV:].unflatten(-1, (H, DV))
    for view, name in zip(views + (gate,), ("q", "k", "v", "gate")):
        view.copy_(torch.from_numpy(d[name]).to(dev).to(torch.bfloat16))
    g = torch.from_numpy(d["g"]).to(dev)
    o = torch.empty((B, T, H, DV), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    fn = lambda: gla.gla_chunk_fwd_strided(*views, g, None, out_dtype=torch.bfloat16, o=o, S_T=S_T)
    ms, _ = _time_calls(torch, fn, steps, warmup, warm_ms=30)
    o_dense, S_dense = gla.gla_chunk_fwd(*(x.contiguous() for x in views), g, None, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    equal = bool(torch.equal(o, o_dense) and torch.equal(S_T, S_dense))
    del o_dense, S_dense
    y = torch.empty_like(o)
    fn_g = lambda: gla.gla_chunk_fwd_strided(*views, g, None, out_dtype=torch.bfloat16, o=y, S_T=S_T, gate=gate)
    ms_g, _ = _time_calls(torch, fn_g, steps, warmup, warm_ms=30)
    torch.cuda.synchronize()
    import oracle
    bs, hs = [0, 7], [0, 15]
    sub = lambda x: x[np.ix_(bs, range(T), hs)]
    y_ref, _ = oracle.forward_gated(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["g"]), sub(d["gate"]))
    nbytes = fwd_bytes(B, T, 2, 2)
    nbytes_g = nbytes + B * T * H * DV * 2                 # the gate read once
    return {"workload": f"prefill B={B} T={T} H=16 bf16 in/out, q, k, v read in place from a [{B}, {T}, 9216] "
                        "fused projection buffer", "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "gated": {"workload": "the same call with the output gate, o * SiLU(gate), the gate read in place "
                                  "from the buffer's fourth part", "ms": ms_g,
                      "tokens_per_s": B * T / (ms_g * 1e-3), "bytes": nbytes_g,
                      "GBps": nbytes_g / (ms_g * 1e-3) / 1e9,
                      "hbm_frac": nbytes_g / (ms_g * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "parity": {"y_bf16_out_over_bound": _bf16_out_ratio(sub(y.float().cpu().numpy()), y_ref, 1e-2),
                                 "sample": "(b,h) in {0,7}x{0,15}, all 2048 tokens"}},
            "parity": {"bitwise_equal_to_dense_call": equal}}


def bench_conv(torch, gla, steps, warmup, B=8, T=2048, D=3072, sets=4):
    """The convolution ahead of the mixer.  Its 201 MB per call would stay in
    the 256 MB last-level cache between repeated calls, so the timed calls
    cycle over `sets` separate input/output pairs (805 MB in all)."""
    dev = torch.device("cuda", 0)
    r = np.random.default_rng(0)
    xs = [torch.from_numpy(gen.bf16_round(r.standard_normal((B, T, D), dtype=np.float32))).to(dev)
          .to(torch.bfloat16) for _ in range(sets)]
    ys = [torch.empty_like(xs[0]) for _ in range(sets)]
    w = torch.from_numpy((r.standard_normal((D, 4)) * 0.5).astype(np.float32)).to(dev)
    bias = torch.from_numpy((r.standard_normal(D) * 0.1).astype(np.float32)).to(dev)
    hist = torch.zeros((B, 4, D), dtype=torch.float32, device=dev)   # each sequence's window, float32
    it = [0]

    def fn():
        i = it[0] % sets
        it[0] += 1
        gla.gla_conv1d_silu(xs[i], w, bias, conv_state=hist, init_from_state=True, y=ys[i])
    ms, _ = _time_calls(torch, fn, steps, warmup, warm_ms=30)
    # sampled parity: sequence 0 of set 0 from a zero window, against the oracle
    import oracle
    hist.zero_()
    gla.gla_conv1d_silu(xs[0], w, bias, conv_state=hist, init_from_state=True, y=ys[0])
    torch.cuda.synchronize()
    x0 = xs[0][0].float().cpu().numpy()
    y_ref, h_ref = oracle.conv1d_silu(x0, w.cpu().numpy(), bias.cpu().numpy(), [0, T], np.zeros((1, 4, D)), None, True)
    parity = {"y_bf16_out_over_bound": _bf16_out_ratio(ys[0][0].float().cpu().numpy(), y_ref, 1e-5),
              "window_bitwise": bool(np.array_equal(hist[0].cpu().numpy(), h_ref[0])),
              "sample": f"sequence 0, all {D} channels, {T} tokens"}
    # x read and y written once (2 B each per token-channel); of each
    # sequence's float32 window three rows read and four written
    nbytes = B * T * D * 4 + B * (3 + 4) * D * 4
    return {"workload": f"causal depth-wise conv1d width 4 + SiLU, B={B} T={T} D={D}, bf16 in/out, "
                        f"float32 window of the last four inputs kept per sequence; calls cycle over {sets} "
                        "input/output sets",
            "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes, "kernels_per_call": 1,
            "parity": parity}


def copy_reference(torch, steps, sets=4, nbytes=100_663_296):
    """What plain streaming reaches on this GPU: torch's device copy of a
    100.7 MB tensor (the size of the prefill's o), cycling over `sets`
    source/destination pairs so that the data comes from HBM."""
    dev = torch.device("cuda", 0)
    src = [torch.randn(nbytes // 4, device=dev) for _ in range(sets)]
    dst = [torch.empty_like(src[0]) for _ in range(sets)]
    it = [0]

    def fn():
        i = it[0] % sets
        it[0] += 1
        dst[i].copy_(src[i])
    ms, _ = _time_calls(torch, fn, steps, 0, warm_ms=30)
    del src, dst
    # the decode's access: one 1.51 GB buffer read and written in place
    S = torch.randn(1280 * 16 * 96 * 192, device=dev)
    ms_ip, _ = _time_calls(torch, lambda: S.mul_(0.999), max(3, steps // 5), 0, warm_ms=30)
    ip_bytes = 2 * S.numel() * 4
    del S
    return {"GBps": 2 * nbytes / (ms * 1e-3) / 1e9, "bytes_per_copy": 2 * nbytes,
            "inplace_GBps": ip_bytes / (ms_ip * 1e-3) / 1e9, "bytes_per_inplace": ip_bytes,
            "note": f"torch device-to-device copy of {nbytes} B (read + write), {sets} rotating pairs; "
                    "torch in-place multiply of the decode's 1.51 GB state (read + write in place); "
                    "reference points, not ceilings"}


def bench_decode(torch, gla, layers=24, steps=64, warmup=1, parity=True, q16=False):
    w = gen.WORKLOADS["decode_1280x24x64"]
    n = w["B"]
    dev = torch.device("cuda", 0)
    S0 = torch.from_numpy(gen.make_decode_state(n, seed=0)).to(dev)
    alloc = gla.gla_state_alloc_q16 if q16 else gla.gla_state_alloc
    pools = [alloc(n) for _ in range(layers)]
    for p in pools:
        gla.gla_state_write(p, S0)
    xs = []
    for s in range(steps):
        x = gen.make_decode_step(n, s, seed=0)
        xs.append(tuple(torch.from_numpy(x[key]).to(dev).to(torch.bfloat16 if key != "g" else torch.float32)
                        for key in ("q", "k", "v", "g")))
    outs = [torch.empty((n, H, DV), dtype=torch.float32, device=dev) for _ in range(layers)]
    # warm-up on the first layer's pool is part of the state history: use a
    # separate scratch pool so the timed run starts from S0 on every layer
    scratch = alloc(n)
    for _ in range(warmup):
        gla.gla_recurrent_step(scratch, *xs[0], out_dtype=torch.float32, o=outs[0])
    torch.cuda.synchronize()
    # events bracket all launches (one step of every layer, steps times); a
    # device spin queued ahead keeps host marshalling out of the timed region
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e6))
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        for l in range(layers):
            gla.gla_recurrent_step(pools[l], *xs[s], out_dtype=torch.float32, o=outs[l])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_launch = ms_total / (steps * layers)
    nbytes = decode_bytes(n, q16=q16)
    state = ("16-bit state (int16 [%d,16,96,192] + an int32 exponent per state column)" % n if q16
             else f"fp32 state [{n},16,96,192]")
    res = {"workload": f"decode step, {n} sequences x {layers} layers x {steps} steps, H=16, "
                       f"{state} per layer, bf16 q/k/v, fp32 o",
           "us_per_layer_step": ms_launch * 1e3, "GBps": nbytes / (ms_launch * 1e-3) / 1e9,
           "hbm_frac": nbytes / (ms_launch * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "tokens_per_s": n * steps / (ms_total * 1e-3), "bytes_per_launch": nbytes,
           "launches": int(steps * layers), "wall_s": wall}
    if parity:
        import oracle
        sample = np.arange(0, n, 80)
        S_ref = gen.make_decode_state(n, seed=0)[sample].astype(np.float64)
        for s in range(steps):
            x = gen.make_decode_step(n, s, seed=0)
            o_ref, S_ref = oracle.step(S_ref, x["q"][sample], x["k"][sample], x["v"][sample], x["g"][sample])
        o_last = outs[0].cpu().numpy()[sample]
        same = all(torch.equal(outs[0], outs[l]) for l in range(1, layers))
        S_got = gla.gla_state_read(pools[0], slot_idx=torch.from_numpy(sample.astype(np.int32)).to(dev)).cpu().numpy()
        # a 16-bit state is compared with the float64 recurrence too: the
        # difference is what the format costs over the steps, not a kernel error
        sfx = "_vs_float64_recurrence" if q16 else ""
        res["parity"] = {"o_last_step" + sfx: _rel_err(o_last, o_ref),
                         f"state_after_{steps}" + sfx: _rel_err(S_got, S_ref),
                         "layers_bitwise_equal": bool(same), "sample": f"{len(sample)} sequences x 16 heads"}
        if q16:
            # the kernel against the oracle from the same stored state: one more
            # (untimed) step on layer 0, o of the sampled sequences
            sl = torch.from_numpy(sample).to(dev)
            m0, e0 = (t[sl].cpu().numpy() for t in pools[0].q16_views())
            gla.gla_recurrent_step(pools[0], *xs[0], out_dtype=torch.float32, o=outs[0])
            x = gen.make_decode_step(n, 0, seed=0)
            o1_ref, _, _ = oracle.step_q16(m0, e0, x["q"][sample], x["k"][sample], x["v"][sample], x["g"][sample])
            res["parity"]["o_one_step_from_stored_state"] = _rel_err(outs[0].cpu().numpy()[sample], o1_ref)
    for p in pools + [scratch]:
        p.free()
    return res


def bench_backward(torch, gla, steps, warmup):
    d = gen.make_inputs("bwd_bf16_b4_t4096", seed=0, with_dO=True)
    B, T = d["meta"]["B"], d["meta"]["T"]
    q, k, v, g, S0, dO = _dev_inputs(torch, d, torch.bfloat16)
    dims = gla.GlaDims(B, T, H, DK, DV, CH, gla.GLA_BF16, gla.GLA_BF16)
    ws = torch.empty(gla.gla_workspace_size(gla.GLA_OP_BWD, dims), dtype=torch.uint8, device=q.device)
    fn = lambda: gla.gla_chunk_bwd(q, k, v, g, dO, out_dtype=torch.bfloat16, workspace=ws)
    ms, _ = _time_calls(torch, fn, steps, warmup, warm_ms=30)
    nbytes = bwd_bytes(B, T, 2, 2)
    flops = BWD_FLOP_PER_TH * B * T * H
    return {"workload": f"backward B={B} T={T} H=16 bf16 in/out, fp32 dg, S0 = dS_T = 0",
            "ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "GBps_algorithmic": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_util": flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
            "mfma_ceiling": mfma_ceiling(flops, nbytes, BF16_PEAK_TFLOPS),
            "kernels_per_call": "5: three launches of the dq, dk and dv walks over two staggered segments, "
                                "partial-sum finish, d-log-decay finish",
            "fp32": bench_backward_f32(torch, gla, steps, warmup)}


def bench_backward_f32(torch, gla, steps, warmup):
    """The backward on fp32 inputs and outputs at the fp32 workload's shape
    (B=1, T=2048, H=16), on the fp32 matrix cores."""
    d = gen.make_inputs("fwd_f32_b1_t2048", seed=0, with_dO=True)
    B, T = d["meta"]["B"], d["meta"]["T"]
    q, k, v, g, S0, dO = _dev_inputs(torch, d, torch.float32)
    dims = gla.GlaDims(B, T, H, DK, DV, CH, gla.GLA_F32, gla.GLA_F32)
    ws = torch.empty(gla.gla_workspace_size(gla.GLA_OP_BWD, dims), dtype=torch.uint8, device=q.device)
    fn = lambda: gla.gla_chunk_bwd(q, k, v, g, dO, out_dtype=torch.float32, workspace=ws)
    ms, _ = _time_calls(torch, fn, steps, warmup, warm_ms=30)
    nbytes = bwd_bytes(B, T, 4, 4)
    flops = BWD_FLOP_PER_TH * B * T * H
    return {"workload": f"backward B={B} T={T} H=16 fp32 in/out, fp32 dg, S0 = dS_T = 0",
            "ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "GBps_algorithmic": nbytes / (ms * 1e-3) / 1e9,
            "mfma_util": flops / (ms * 1e-3) / (F32_MFMA_PEAK_TFLOPS * 1e12), "mfma_peak": f"fp32 {F32_MFMA_PEAK_TFLOPS} TFLOP/s",
            "kernels_per_call": "state-only walks of both recurrences, 2 segment scans, 4 dq/dk walks, the dv walk, "
                                "row dots, partial-sum finish, d-log-decay finish"}


def src_digest():
    """Digest of the sources the prefill walk kernel is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_simple_amd", "csrc")
    for name in ("gla_common.h", "gla_kernels.h", "gla_walk.hip"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles():
    """HBM bytes per prefill launch from the committed counter summary, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "prefill_walk_b8_t2048_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            key, _, val = line[2:].partition(":")
            vals[key.strip()] = val.strip()
    if vals.get("kernel_source_digest") != src_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--only", choices=["prefill", "decode", "decode_q16", "backward", "packed", "conv", "fused", "prefix", "probe",
                                       "long", "copy"],
                    default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs the mixer on a single MI355X and has no "
              "multi-GPU path (every (b, h) is independent, so the prefill, decode and backward would "
              "shard over batch or heads with no exchange). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.only:
        torch, gla = _gpu()
        if args.only == "prefill":
            print(json.dumps(bench_prefill(torch, gla, args.steps, args.warmup, parity=False)))
        elif args.only == "decode":
            print(json.dumps(bench_decode(torch, gla, layers=1, steps=args.steps, warmup=args.warmup,
                                          parity=False)))
        elif args.only == "decode_q16":
            print(json.dumps(bench_decode(torch, gla, layers=1, steps=args.steps, warmup=args.warmup,
                                          parity=False, q16=True)))
        elif args.only == "backward":
            print(json.dumps(bench_backward(torch, gla, args.steps, args.warmup)))
        elif args.only == "packed":
            print(json.dumps(bench_packed(torch, gla, args.steps, args.warmup)))
        elif args.only == "conv":
            print(json.dumps(bench_conv(torch, gla, args.steps, args.warmup)))
        elif args.only == "fused":
            print(json.dumps(bench_fused(torch, gla, args.steps, args.warmup)))
        elif args.only == "probe":
            print(json.dumps({"device": device_probe(torch), "mall": bench_prefill_mall_warm(torch, gla, args.steps)}))
        elif args.only == "prefix":
            print(json.dumps(bench_decode_after_prefix(torch, gla)))
        elif args.only == "long":
            print(json.dumps(bench_prefill_other(torch, gla, "fwd_bf16_b1_t65536", torch.bfloat16, torch.bfloat16,
                                                 args.steps, args.warmup)))
        else:
            n = 1 << 28
            a = torch.ones(n, dtype=torch.float32, device="cuda")
            b = torch.empty_like(a)
            for _ in range(args.warmup + args.steps):
                b.copy_(a)
            torch.cuda.synchronize()
            print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                              "launches": args.warmup + args.steps}))
        return

    cpu = None if args.no_cpu else cpu_baseline()       # before any GPU work
    print(f"[bench] cpu baseline done", file=sys.stderr, flush=True)
    cpu_dec = None if args.no_cpu else cpu_decode_baseline()
    print(f"[bench] cpu decode baseline done", file=sys.stderr, flush=True)
    torch, gla = _gpu()
    torch.cuda.synchronize()
    pre = bench_prefill(torch, gla, args.steps, args.warmup)
    print(f"[bench] prefill {pre['ms']:.4f} ms", file=sys.stderr, flush=True)
    dec = bench_decode(torch, gla)
    print(f"[bench] decode {dec['us_per_layer_step']:.1f} us/layer-step", file=sys.stderr, flush=True)
    dec16 = bench_decode(torch, gla, q16=True)
    print(f"[bench] decode, 16-bit state {dec16['us_per_layer_step']:.1f} us/layer-step", file=sys.stderr, flush=True)
    bwd = bench_backward(torch, gla, max(3, args.steps // 2), 2)
    print(f"[bench] backward {bwd['ms']:.4f} ms", file=sys.stderr, flush=True)
    lc = bench_prefill_other(torch, gla, "fwd_bf16_b1_t65536", torch.bfloat16, torch.bfloat16,
                             max(3, args.steps // 2), 2)
    f32 = bench_prefill_other(torch, gla, "fwd_f32_b1_t2048", torch.float32, torch.float32,
                              max(3, args.steps // 2), 2)
    packed = bench_packed(torch, gla, max(3, args.steps // 2), 2)
    print(f"[bench] packed {packed['ms']:.4f} ms", file=sys.stderr, flush=True)
    fused = bench_fused(torch, gla, args.steps, args.warmup)
    print(f"[bench] fused {fused['ms']:.4f} ms", file=sys.stderr, flush=True)
    conv = bench_conv(torch, gla, max(3, args.steps // 2), 2)
    pfx = bench_decode_after_prefix(torch, gla)
    print(f"[bench] decode after 2,048 / 8,192-token prefixes: {pfx['us_per_step_after_2048_tokens']:.1f} / "
          f"{pfx['us_per_step_after_8192_tokens']:.1f} us", file=sys.stderr, flush=True)
    mall = bench_prefill_mall_warm(torch, gla, args.steps)
    print(f"[bench] prefill, inputs just written {mall['ms_inputs_just_written']:.4f} ms", file=sys.stderr,
          flush=True)
    copy = copy_reference(torch, args.steps)
    mref = mfma_reference(torch)
    probe = device_probe(torch)
    print(f"[bench] conv {conv['ms']:.4f} ms", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC, "value": pre["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pre["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "chunked prefill B=8 T=2048 H=16 dk=96 dv=192 chunk=128, bf16 q/k/v/o, "
                               "fp32 log-decay/state/accumulation, log-decay logsigmoid(N(0,1)+4), S0=0",
                   "global_batch": 8, "seq_len": 2048, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": pre["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pre["GBps"] / HBM_PEAK_GBS, "traffic": traffic_from_profiles(),
                     "kernel": "walk_kernel<bf16,bf16,3,0,false> (gla_chunk_fwd)",
                     "algorithmic_bytes_per_launch": pre["bytes"]},
        "mfma_util": {"value": pre["mfma_util"], "algorithmic_flop_per_step": pre["flops"],
                      "peak": "bf16 dense 2500 TFLOP/s", "ceiling": pre["mfma_ceiling"],
                      "value_over_ceiling": pre["mfma_util"] / pre["mfma_ceiling"],
                      "measured_gemm_reference": mref,
                      "note": "dense 128-token chunks; ceiling = what the HBM roof allows for this "
                              "workload's algorithmic bytes and FLOPs"},
        "prefill_mall_warm": mall,
        "device": probe,
        "decode_after_prefix": pfx,
        "decode": dec, "decode_q16": dec16, "backward": bwd, "long_context": lc, "fp32": f32, "packed": packed, "fused": fused, "conv": conv,
        "parity": {"prefill": pre.get("parity")},
        "hbm_copy_reference": dict(copy, prefill_frac_of_copy=pre["GBps"] / copy["GBps"],
                                   decode_frac_of_copy=dec["GBps"] / copy["GBps"],
                                   decode_frac_of_inplace=dec["GBps"] / copy["inplace_GBps"],
                                   decode_q16_frac_of_inplace=dec16["GBps"] / copy["inplace_GBps"],
                                   conv_frac_of_copy=conv["GBps"] / copy["GBps"]),
        "cpu_baseline": cpu,
        "cpu_baseline_decode": cpu_dec,
        "kernel_source_digest": src_digest(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
