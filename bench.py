#!/usr/bin/env python3
"""KDA forward benchmark on one MI355X.

Workload (one timed step): the chunked prefill of one 32768-token sequence,
32 heads, dk = dv = 128, 64-token chunks, bf16 q/k/v/beta/o, fp32 g, a nonzero
fp32 initial state and fp32 final state -- the prefill-32k workload.  Beside it
the recurrent decode leg: batch 64, 32 heads, d = 128, 256 successive
one-token steps on a carried state produced by a chunked prefill of 1024
tokens per sequence.

Further legs beside it: the prefill with the gate activation fused, a
continuing prefill (16 new tokens per sequence through the recurrent op), and
the short causal conv (forward over the prefill-32k tokens, one-token update
at the decode shape).  Decode steps and conv updates are also captured once in
a graph and replayed (each replay checked bit for bit against the eager run):
the replay time is the kernels' own, the eager time beside it includes the
per-call host cost of issuing them one by one from Python.

Prints one JSON line.  `value` is prefill tokens/s with inputs resident in HBM.
The roofline entry prices the prefill against HBM bandwidth with the
algorithmic bytes of the pass (q, k, v, g, beta read once, o written once, h0
read and hT written); per-kernel durations come from HIP events recorded on the
launch stream around each of the three launches.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
# The CPU oracle (OpenMP) runs last; its idle threads sleep instead of
# spinning on the cores the GPU legs' host thread uses.
os.environ.setdefault("OMP_WAIT_POLICY", "PASSIVE")

METRIC = "KDA prefill tokens/s (H=32,d=128,T=32k) + decode steps/s; % of roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

# Algorithmic traffic per token, bf16 inputs, H = 32, d = 128: q, k, v (bf16),
# g (fp32), beta (bf16) read once, o (bf16) written once.
BYTES_PER_TOKEN = 3 * 8192 + 16384 + 64 + 8192  # 49,216
# With the gate fused: g (fp32, 16,384 B/token) is replaced by the raw gate x (bf16).
BYTES_PER_TOKEN_GATED = 3 * 8192 + 8192 + 64 + 8192  # 41,024
STATE_BYTES = 32 * 128 * 128 * 4  # one sequence's h0 or hT
# The same bytes split by stage: the chunk-local stage reads q, k, v, g, beta;
# the state scan writes o and reads h0 / writes hT (the workspace between
# them is not algorithmic traffic).
LOCAL_BYTES_PER_TOKEN = 3 * 8192 + 16384 + 64  # 41,024
SCAN_BYTES_PER_TOKEN = 8192
# Algorithmic flops per (64-token chunk, head) of the chunked form.
FLOPS_PER_CHUNK_HEAD = 9_041_236
# Decode: state read + written per step, plus the step's q, k, v, g, beta, o.
DECODE_STATE_BYTES = 64 * 32 * 128 * 128 * 4 * 2
DECODE_TOKEN_BYTES = 64 * 32 * (128 * 2 * 3 + 128 * 4 + 2 + 128 * 2)
DECODE_FLOPS = 64 * 32 * (7 * 128 * 128)

COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = ["gated_delta_rule_55_amd/csrc/kda_prefill.hip",
                  "gated_delta_rule_55_amd/csrc/kda_headscan.hip",
                  "gated_delta_rule_55_amd/csrc/kda_conv.hip",
                  "gated_delta_rule_55_amd/csrc/kda_chunk_ops.h",
                  "gated_delta_rule_55_amd/csrc/kda_decode.hip",
                  "gated_delta_rule_55_amd/csrc/kda_device.h",
                  "gated_delta_rule_55_amd/build.py"]  # its flags shape the kernels too


def _code_only(rel: str, text: str) -> str:
    """The HIP sources without their comments and with every run of white space
    read as one space (a comment or layout edit does not change a kernel, so it
    must not retire the counters taken on it)."""
    if not rel.endswith((".hip", ".h")):
        return text
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(rel, f.read()).encode())
    return h.hexdigest()[:16]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_counter(kernel: str, field: str):
    """A per-launch figure from committed counter runs, or None when absent or
    taken on a different version of the kernel sources."""
    try:
        with open(COUNTERS_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("source_hash") != kernel_source_hash():
        return None
    ent = data.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get(field)


def measured_traffic(kernel: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a copy)."""
    return measured_counter(kernel, "bytes_per_launch")


def to_dev(arr, torch):
    import numpy as np

    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(arr).cuda()


def bench_prefill(args, torch, kda, synth, inp=None, fused_gate=False):
    """Time the prefill-32k pass.  fused_gate: pass the raw gate (x bf16,
    a_log, dt_bias) instead of g, so the kernels compute the gate activation."""
    if inp is None:
        log("generating the prefill-32k inputs (seeded numpy)")
        inp = synth.make_config(2)
    T, H, D = inp.T, inp.H, inp.dk
    N = len(inp.cu_seqlens) - 1
    q, k, v = (to_dev(x, torch) for x in (inp.q, inp.k, inp.v))
    beta = to_dev(inp.beta, torch)
    cu = None if N == 1 else torch.from_numpy(inp.cu_seqlens).cuda()
    if fused_gate:
        g = None
        gate = (to_dev(inp.gate_x, torch), to_dev(inp.gate_a_log, torch),
                to_dev(inp.gate_dt_bias, torch))
    else:
        g, gate = to_dev(inp.g, torch), None
    h0 = None if inp.h0 is None else to_dev(inp.h0, torch)
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.prefill_workspace_bytes(T, H, D, N, 64), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for row in ev:  # create the underlying events
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()

    def run(events=None):
        kda.chunk_prefill(q, k, v, g, beta, h0, cu, scale=inp.scale, chunk=64, out=o, ht=ht,
                          workspace=ws, events=events, plan=args.plan, gate=gate)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        run(ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # events: before the chunk map, after it, after the chunk-local stage,
    # after the state scan
    stage = {"chunk_map": [], "chunk_local": [], "state_scan": [], "prefill_call": []}
    for row in ev:
        stage["chunk_map"].append(row[0].elapsed_time(row[1]))
        stage["chunk_local"].append(row[1].elapsed_time(row[2]))
        stage["state_scan"].append(row[2].elapsed_time(row[3]))
        stage["prefill_call"].append(row[0].elapsed_time(row[3]))
    avg = {kname: statistics.mean(vals) for kname, vals in stage.items()}
    ms_per_step = total_ms / args.steps
    return inp, ms_per_step, avg


def bench_prefill_batch(args, torch, kda, synth, cfg, full=None):
    """Batched prefills: the packed varlen batch (8 sequences, lengths in
    [300, 8192], h0 given) and the 64 x 1024-token prefill that seeds the
    decode leg (no h0).  Wider scan blocks apply here (many sequence-heads)."""
    if cfg == 3:
        log("generating the varlen-8 prefill inputs (seeded numpy)")
        inp = synth.make_config(3)
        name = "varlen-8: 8 packed sequences, lengths seeded in [300, 8192]"
    else:
        N, L, P = 64, 1280, 1024
        rows = np.concatenate([np.arange(n * L, n * L + P) for n in range(N)])
        inp = synth.KdaInputs(**{**full.__dict__, **{
            f: getattr(full, f)[rows] for f in ("q", "k", "v", "g", "beta", "gate_x")
            if getattr(full, f) is not None},
            "cu_seqlens": np.arange(0, N * P + 1, P, dtype=np.int32)})
        name = "64 x 1024: the prefill that seeds the decode leg"
    _, ms_step, stage = bench_prefill(args, torch, kda, synth, inp=inp)
    T, N = inp.T, len(inp.cu_seqlens) - 1
    nstate = N * (2 if inp.h0 is not None else 1)
    alg = T * BYTES_PER_TOKEN + nstate * STATE_BYTES
    ach = alg / (stage["prefill_call"] / 1e3) / 1e9
    return {"workload": name + f", {T} tokens, H=32, d=128, chunk 64, bf16",
            "tokens_per_s": round(T / (ms_step / 1e3), 1), "ms_per_step": round(ms_step, 4),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                         "scope": f"whole prefill pass, {alg} algorithmic bytes per pass"},
            "kernels_ms": {kname: round(v, 4) for kname, v in stage.items()}}


def bench_prefill_4k(args, torch, kda, synth, reps=10):
    """The prefill-4k workload (1 sequence x 4096 tokens, H=32, d=128, no h0):
    warm, back to back (its 204 MB of inputs and outputs fit the 256 MB
    Infinity Cache), and cold, each pass timed alone right after a 512 MB
    scratch read outside the timed region."""
    log("generating the prefill-4k inputs (seeded numpy)")
    inp = synth.make_config(1)
    T, H, D = inp.T, inp.H, inp.dk
    q, k, v = (to_dev(x, torch) for x in (inp.q, inp.k, inp.v))
    beta, g = to_dev(inp.beta, torch), to_dev(inp.g, torch)
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.prefill_workspace_bytes(T, H, D, 1, 64), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    flush = _flusher(torch)

    def run():
        kda.chunk_prefill(q, k, v, g, beta, None, None, scale=inp.scale, chunk=64, out=o, ht=ht,
                          workspace=ws)

    def timed(pre=None):
        if pre:
            pre()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    warm = statistics.median([timed() for _ in range(reps)])
    cold = statistics.median([timed(flush) for _ in range(reps)])
    alg = T * BYTES_PER_TOKEN + STATE_BYTES
    res = {"workload": "prefill-4k: 1 sequence x 4096 tokens, H=32, dk=dv=128, chunk 64, bf16 "
                       "q/k/v/beta/o, fp32 g, no h0",
           "warm": {"ms_per_pass": round(warm, 4), "tokens_per_s": round(T / (warm / 1e3), 1),
                    "frac": round(alg / (warm / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
           "cold": {"ms_per_pass": round(cold, 4), "tokens_per_s": round(T / (cold / 1e3), 1),
                    "frac": round(alg / (cold / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
           "note": f"{alg} algorithmic bytes per pass; each pass timed alone (HIP events around "
                   f"the call), median of {reps}; cold passes follow a {FLUSH_BYTES >> 20} MB "
                   "scratch read, warm ones follow the previous pass"}
    del q, k, v, beta, g, o, ws
    return res


def bench_decode(args, torch, kda, synth, inp):
    N, L, P, S = 64, 1280, 1024, args.decode_steps
    H, D = inp.H, inp.dk
    dev = {name: to_dev(getattr(inp, name), torch) for name in ["q", "k", "v", "g", "beta"]}
    view = lambda t: t.view(N, L, *t.shape[1:])  # noqa: E731
    pre = {kk: view(t)[:, :P].reshape(N * P, *t.shape[1:]).contiguous() for kk, t in dev.items()}
    dec = {kk: view(t)[:, P:P + S].transpose(0, 1).contiguous() for kk, t in dev.items()}
    del dev
    cu = torch.arange(0, N * P + 1, P, dtype=torch.int32, device="cuda")
    _, state0 = kda.chunk_prefill(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], None, cu,
                                  scale=inp.scale, chunk=64)
    out = torch.empty((S, N, H, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    eager, ms = _decode_steps_timed(args, torch, kda, inp, state0, dec, out, stream)
    # the same steps on a bf16 copy of the state (half the state bytes)
    eager16, ms16 = _decode_steps_timed(args, torch, kda, inp, state0.to(torch.bfloat16), dec,
                                        out, stream)
    cold = _decode_cold(torch, kda, inp, state0, dec, stream)
    rec = bench_recurrent(args, torch, kda, inp, state0, dec, stream)
    rec["eager_decode_ms_per_step"] = round(eager / S, 5)
    rec["bf16_state"] = {"ms": ms16, "eager_ms_per_step": round(eager16 / S, 5)}
    return inp, S, ms, dec, rec, state0, cold


def _decode_steps_timed(args, torch, kda, inp, state0, dec, out, stream):
    """S decode steps from state0: median eager time (one Python call per
    step) and median time of the same steps replayed from a captured graph,
    as a serving loop issues decode (the kernels' own time, without per-call
    host cost).  Each replay is checked bit for bit against the eager run."""
    S = out.shape[0]
    state = state0.clone()

    def steps():
        for s in range(S):
            kda.recurrent_decode(state, dec["q"][s], dec["k"][s], dec["v"][s], dec["g"][s],
                                 dec["beta"][s], scale=inp.scale, out=out[s])

    def timed(fn):
        state.copy_(state0)  # restore, untimed
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    state.copy_(state0)
    steps()  # warm-up
    eager = [timed(steps) for _ in range(args.decode_reps)]
    out_ref, state_ref = out.clone(), state.clone()
    graph = torch.cuda.CUDAGraph()
    state.copy_(state0)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            steps()
    times = []
    for _ in range(max(3, args.decode_reps)):
        times.append(timed(graph.replay))
        if not (torch.equal(state, state_ref) and torch.equal(out, out_ref)):
            raise RuntimeError("graph replay of the decode steps differs from the eager run")
    return statistics.median(eager), statistics.median(times)


FLUSH_BYTES = 512 << 20  # twice the 256 MB Infinity Cache


def _flusher(torch, device="cuda", nbytes=FLUSH_BYTES):
    """A 512 MB buffer whose read (a sum), issued between timed launches,
    leaves the Infinity Cache holding only its own lines.  A read rather than a
    fill, so the lines it leaves are clean: the timed launch that follows does
    not pay for writing a scratch buffer back to HBM."""
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    res = torch.empty((), dtype=torch.float32, device=device)

    def flush():
        torch.sum(buf, dim=0, out=res)
    return flush


def _decode_cold(torch, kda, inp, state0, dec, stream, n=32):
    """Decode steps with the Infinity Cache flushed before each: n x (512 MB
    scratch read, step) back to back between two events, minus n reads alone,
    divided by n -- each step then reads the state and its inputs from HBM
    (and the write-back of the state it wrote falls in the difference).
    The back-to-back steps of the main leg keep the 134 MB state in the
    256 MB Infinity Cache instead."""
    flush = _flusher(torch)
    S = next(iter(dec.values())).shape[0]
    state = state0.clone()
    out = torch.empty((state.shape[0], inp.H, inp.dk), dtype=torch.bfloat16, device="cuda")

    def span(with_step):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            flush()
            if with_step:  # the drawn decode tokens in turn, again from the first if n > S
                s = i % S
                kda.recurrent_decode(state, dec["q"][s], dec["k"][s], dec["v"][s], dec["g"][s],
                                     dec["beta"][s], scale=inp.scale, out=out)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    span(True)  # warm-up
    both = statistics.median([span(True) for _ in range(3)])
    fills = statistics.median([span(False) for _ in range(3)])
    return {"cold_ms": (both - fills) / n, "fill_ms": fills / n, "n": n}


def bench_recurrent(args, torch, kda, inp, state0, dec, stream, R=16):
    """Continuing prefill: the next R tokens of all 64 sequences in one
    recurrent-prefill call on the carried state (a state pool, slot n for
    sequence n), against R decode steps doing the same work."""
    N, H, D = state0.shape[0], inp.H, inp.dk
    R = min(R, next(iter(dec.values())).shape[0])  # no more tokens than the decode steps drew
    packed = {kk: t[:R].transpose(0, 1).reshape(N * R, *t.shape[2:]).contiguous()
              for kk, t in dec.items()}
    cu = torch.arange(0, N * R + 1, R, dtype=torch.int32, device="cuda")
    slots = torch.arange(N, dtype=torch.int32, device="cuda")
    pool = state0.clone()
    out = torch.empty((N * R, H, D), dtype=torch.bfloat16, device="cuda")

    def call():
        kda.recurrent_prefill(packed["q"], packed["k"], packed["v"], packed["g"], packed["beta"],
                              pool, cu, scale=inp.scale, out=out, ht=pool, state_indices=slots)

    call()  # warm-up
    times = []
    for _ in range(max(3, args.decode_reps)):
        pool.copy_(state0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = statistics.median(times)
    rbytes = DECODE_STATE_BYTES + R * DECODE_TOKEN_BYTES
    ach = rbytes / (ms / 1e3) / 1e9
    return {"workload": f"continuing prefill: {R} new tokens for each of 64 sequences (H=32, "
                        "d=128) on the carried decode-leg state, one recurrent-prefill call "
                        "over a 64-slot state pool",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(N * R / (ms / 1e3), 1),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                         "scope": f"state read + write once and {R} tokens' inputs and outputs, "
                                  f"{rbytes} bytes per call"}}


CONV_DIM = 3 * 32 * 128  # [q|k|v] channels at H = 32, d = 128
CONV_W = 4


def bench_conv(args, torch, kda, T=32768, N_dec=64, reps=10, dec_calls=256):
    """The short causal conv over the [q|k|v] channels (dim 12288, W = 4, SiLU,
    bf16) that feeds the prefill: the varlen forward over the prefill-32k
    tokens writing q, k, v as separate tensors and the new taps, then the
    one-token update at the decode shape (64 sequences, 64-slot tap pool).
    Inputs: N(0, 1) activations and taps, U(-1/2, 1/2) weight and bias, drawn
    with a seeded device generator."""
    dim, W = CONV_DIM, CONV_W
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    x = torch.randn((T, dim), generator=gen, device="cuda").to(torch.bfloat16)
    w = torch.rand((dim, W), generator=gen, device="cuda") - 0.5
    b = torch.rand((dim,), generator=gen, device="cuda") - 0.5
    st0 = torch.randn((1, W - 1, dim), generator=gen, device="cuda").to(torch.bfloat16)
    st = st0.clone()
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    outs = tuple(torch.empty((T, dim // 3), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    stream = torch.cuda.current_stream()

    def fwd():
        kda.causal_conv1d_fwd(x, w, b, cu, st0, st, split=(dim // 3,) * 3, out=outs)

    for _ in range(3):
        fwd()
    # back-to-back calls between the events keep the GPU busy, so the host's
    # enqueue time of a call is not counted
    times = []
    for _ in range(reps):
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(10):
            fwd()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(e) / 10)
    ms = statistics.median(times)
    fbytes = 2 * T * dim * 2 + 2 * (W - 1) * dim * 2 + dim * (W + 1) * 4
    fach = fbytes / (ms / 1e3) / 1e9
    res = {"workload": f"causal conv forward over the prefill-32k tokens: T={T}, dim={dim} "
                       f"([q|k|v], H=32, d=128), W={W}, SiLU, bf16, q/k/v written as separate "
                       "tensors, carried taps in and out",
           "ms_per_call": round(ms, 4), "tokens_per_s": round(T / (ms / 1e3), 1),
           "roofline": {"bound": "hbm", "achieved": round(fach, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(fach / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("conv"),
                        "scope": f"x read once, y written once, taps, weight and bias: "
                                 f"{fbytes} bytes per call (both launches)"}}
    del x, outs
    # decode shape: one token for each of 64 sequences per call
    xd = torch.randn((dec_calls, N_dec, dim), generator=gen, device="cuda").to(torch.bfloat16)
    pool0 = torch.randn((N_dec, W - 1, dim), generator=gen, device="cuda").to(torch.bfloat16)
    pool = pool0.clone()
    slots = torch.arange(N_dec, dtype=torch.int32, device="cuda")
    yd = tuple(torch.empty((N_dec, dim // 3), dtype=torch.bfloat16, device="cuda")
               for _ in range(3))

    def updates():
        for i in range(dec_calls):
            kda.causal_conv1d_update(xd[i], w, b, pool, state_indices=slots,
                                     split=(dim // 3,) * 3, out=yd)

    updates()  # warm-up
    pool.copy_(pool0)
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    a.record(stream)
    updates()  # issued from Python, one call at a time
    e.record(stream)
    torch.cuda.synchronize()
    host_us = (time.perf_counter() - h0) * 1e6 / dec_calls
    eager_us = a.elapsed_time(e) * 1e3 / dec_calls
    y_ref = tuple(t.clone() for t in yd)
    pool_ref = pool.clone()
    # The same calls captured once in a graph and replayed: the kernels' own
    # time, without the per-call host cost.  Every replay is checked against
    # the eager run.
    graph = torch.cuda.CUDAGraph()
    pool.copy_(pool0)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            updates()
    times = []
    for _ in range(3):
        pool.copy_(pool0)
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(e))
        if not (torch.equal(pool, pool_ref) and all(torch.equal(x, r) for x, r in zip(yd, y_ref))):
            raise RuntimeError("graph replay of the conv updates differs from the eager run")
    ums = statistics.median(times) / dec_calls
    ubytes = 2 * N_dec * dim * 2 + 2 * N_dec * (W - 1) * dim * 2 + dim * (W + 1) * 4
    uach = ubytes / (ums / 1e3) / 1e9
    res["update"] = {
        "workload": f"causal conv one-token update: {N_dec} sequences, dim={dim}, W={W}, SiLU, "
                    f"bf16, {N_dec}-slot tap pool; {dec_calls} calls replayed from a captured "
                    "graph (checked bitwise against the eager run)",
        "us_per_call": round(ums * 1e3, 2),
        "eager_us_per_call": round(eager_us, 2), "eager_host_us_per_call": round(host_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(uach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(uach / HBM_PEAK_GBS, 4), "traffic": None,
                     "scope": f"{ubytes} bytes per call; launch-bound at this size"}}
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_runs(fn, runs=3):
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times), times


def cpu_prefill_baseline(args, inp):
    """The fp64 oracle (C, OpenMP over the 32 head chains) on the prefill-32k
    inputs: all host threads over the whole sequence, median of 3 runs; and
    one thread over a sample of the heads (the chains are independent and
    equal in work, so tokens/s at 32 heads scales by the sampled fraction),
    median of 3 runs."""
    import oracle

    f = inp.f64()
    threads = oracle.num_threads()
    med, runs = _median_runs(lambda: oracle.prefill(f["q"], f["k"], f["v"], f["g"], f["beta"],
                                                    f["h0"], None, f["scale"]))
    heads = [0, 11, 22]
    sub = synth_slice(inp, heads).f64()
    oracle.set_num_threads(1)
    try:
        med1, runs1 = _median_runs(lambda: oracle.prefill(sub["q"], sub["k"], sub["v"], sub["g"],
                                                          sub["beta"], sub["h0"], None,
                                                          sub["scale"]))
    finally:
        oracle.set_num_threads(threads)
    frac = len(heads) / inp.H
    return {"value": round(inp.T / med, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"fp64 token recurrence over all {inp.T} tokens x {inp.H} heads of the "
                      f"prefill-32k inputs (with h0), {threads} threads, median of 3 runs "
                      f"({', '.join(f'{t:.2f}' for t in runs)} s)",
            "single_thread": {"value": round(inp.T * frac / med1, 1), "unit": "tokens/s",
                              "cores": 1,
                              "sample": f"heads {heads} of the same inputs, one thread, median of "
                                        f"3 runs ({', '.join(f'{t:.2f}' for t in runs1)} s); "
                                        f"tokens/s at {inp.H} heads = T x {len(heads)}/{inp.H} / "
                                        "time"}}


def synth_slice(inp, heads):
    import synth

    return synth.slice_heads(inp, heads)


def cpu_decode_baseline(inp, dec, state0, n_steps=32, n_steps_1t=4):
    """The fp64 oracle's decode step at batch 64 from the carried decode-leg
    state (the GPU's chunked prefill of 1024 tokens per sequence), all host
    threads over n_steps steps and one thread over n_steps_1t steps, each the
    median of 3 runs."""
    import numpy as np

    import oracle

    st0 = state0.double().cpu().numpy()
    arrs = {kk: t[:n_steps].float().cpu().numpy().astype(np.float64) for kk, t in dec.items()}

    def steps(n):
        st = st0
        for s in range(n):
            _, st = oracle.decode(st, arrs["q"][s], arrs["k"][s], arrs["v"][s], arrs["g"][s],
                                  arrs["beta"][s], inp.scale)

    threads = oracle.num_threads()
    med, runs = _median_runs(lambda: steps(n_steps))
    oracle.set_num_threads(1)
    try:
        med1, runs1 = _median_runs(lambda: steps(n_steps_1t))
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(n_steps / med, 2), "unit": "steps/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{n_steps} fp64 decode steps at batch 64, H=32, d=128 from the carried "
                      f"state, {threads} threads, median of 3 runs "
                      f"({', '.join(f'{t:.2f}' for t in runs)} s)",
            "single_thread": {"value": round(n_steps_1t / med1, 3), "unit": "steps/s", "cores": 1,
                              "sample": f"{n_steps_1t} steps, one thread, median of 3 runs "
                                        f"({', '.join(f'{t:.2f}' for t in runs1)} s)"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-reps", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg")
    ap.add_argument("--no-batch", action="store_true",
                    help="skip the batched prefill legs (varlen-8, 64 x 1024)")
    ap.add_argument("--no-gate", action="store_true", help="skip the fused-gate prefill leg")
    ap.add_argument("--no-conv", action="store_true", help="skip the causal conv leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--plan", choices=["auto", "two_pass"], default="auto",
                    help="prefill launch plan")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the KDA path shards by heads or sequences with no communication; "
              "the benchmark runs and reports a single GPU)", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gated_delta_rule_55_amd as kda
    import synth

    inp, ms_step, stage_ms = bench_prefill(args, torch, kda, synth)
    T, H, D = inp.T, inp.H, inp.dk
    tok_s = T / (ms_step / 1e3)
    alg_bytes = T * BYTES_PER_TOKEN + 2 * STATE_BYTES
    n_chunks = (T + 63) // 64
    alg_flops = n_chunks * H * FLOPS_PER_CHUNK_HEAD
    call_ms = stage_ms["prefill_call"]
    achieved = alg_bytes / (call_ms / 1e3) / 1e9
    traffic = measured_traffic("prefill")
    mfma_cnt = measured_counter("prefill", "mfma_bf16_flop_per_launch")
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "scope": "whole prefill pass (chunk map + chunk-local + state scan), "
                 f"{alg_bytes} algorithmic bytes per pass",
        "mfma_frac": round(alg_flops / (call_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        # bf16 MFMA flops the kernels issue per pass (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)
        "mfma_frac_counters": (None if mfma_cnt is None else
                               round(mfma_cnt / (call_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)),
        "kernels_ms": {kname: round(v, 4) for kname, v in stage_ms.items()},
        "plan": args.plan,
    }
    # Each stage against its own algorithmic bytes and its own event-timed
    # duration (HIP events on the launch stream around each launch), with the
    # stage's counter traffic; "dominant" is the longer stage.
    stage_alg = {"chunk_local": T * LOCAL_BYTES_PER_TOKEN,
                 "state_scan": T * SCAN_BYTES_PER_TOKEN + 2 * STATE_BYTES}
    stages = {}
    for kname, kb in stage_alg.items():
        kach = kb / (stage_ms[kname] / 1e3) / 1e9
        stages[kname] = {"achieved": round(kach, 1), "frac": round(kach / HBM_PEAK_GBS, 4),
                         "ms": round(stage_ms[kname], 4), "algorithmic_bytes": kb,
                         "traffic": measured_traffic(kname)}
    dom = max(stages, key=lambda kn: stage_ms[kn])
    roofline["dominant_kernel"] = dom
    roofline["dominant"] = dict(kernel=dom, bound="hbm", peak=HBM_PEAK_GBS, unit="GB/s",
                                **stages[dom])
    roofline["stages"] = stages
    line = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill-32k: 1 sequence x 32768 tokens, H=32, dk=dv=128, "
                               "chunk 64, bf16 q/k/v/beta/o, fp32 g, h0 ~ N(0, 0.02) fp32",
                   "global_batch": 1, "seq_len": T, "heads": H, "head_dim": D, "chunk": 64,
                   "parallelism": "single GPU"},
        "roofline": roofline,
    }
    if not args.no_gate:
        # the same workload with the gate activation fused into the kernels:
        # the pass reads the raw gate x (bf16) instead of g (fp32)
        _, gms_step, gstage = bench_prefill(args, torch, kda, synth, inp=inp, fused_gate=True)
        gbytes = T * BYTES_PER_TOKEN_GATED + 2 * STATE_BYTES + H * 4 + H * D * 4
        gach = gbytes / (gstage["prefill_call"] / 1e3) / 1e9
        line["fused_gate"] = {
            "workload": "prefill-32k with the gate activation fused: raw gate x bf16 "
                        "[T, H, dk], a_log fp32 [H], dt_bias fp32 [H, dk] instead of g fp32",
            "tokens_per_s": round(T / (gms_step / 1e3), 1), "ms_per_step": round(gms_step, 4),
            "roofline": {"bound": "hbm", "achieved": round(gach, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gach / HBM_PEAK_GBS, 4), "traffic": None,
                         "scope": f"whole prefill pass, {gbytes} algorithmic bytes per pass"},
            "kernels_ms": {kname: round(v, 4) for kname, v in gstage.items()},
        }
    if not args.no_batch:
        line["prefill_4k"] = bench_prefill_4k(args, torch, kda, synth)
    inp4 = None
    if not (args.no_batch and args.no_decode):
        log("generating the decode-64x256 inputs (seeded numpy)")
        inp4 = synth.make_config(4)
    if not args.no_batch:
        line["prefill_batches"] = [bench_prefill_batch(args, torch, kda, synth, 3),
                                   bench_prefill_batch(args, torch, kda, synth, 4, inp4)]
    if not args.no_decode:
        dinp, S, dms, dec, rec, dstate0, cold = bench_decode(args, torch, kda, synth, inp4)
        step_ms = dms / S
        dbytes = DECODE_STATE_BYTES + DECODE_TOKEN_BYTES
        dach = dbytes / (step_ms / 1e3) / 1e9
        line["decode"] = {
            "workload": "decode-64x256: batch 64, H=32, d=128, 256 steps on a state from a "
                        "64 x 1024-token chunked prefill, the steps replayed from a captured "
                        "graph (checked bitwise against the eager run)",
            "steps_per_s": round(1e3 / step_ms, 1), "ms_per_step": round(step_ms, 5),
            "eager_ms_per_step": rec.pop("eager_decode_ms_per_step"),
            "tokens_per_s": round(64 * 1e3 / step_ms, 1),
            "roofline": {"bound": "hbm", "achieved": round(dach, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(dach / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode"),
                         "note": "back-to-back steps: the 134 MB state stays in the 256 MB "
                                 "Infinity Cache between steps, so this fraction includes "
                                 "Infinity Cache hits; see cold"},
        }
        cach = dbytes / (cold["cold_ms"] / 1e3) / 1e9
        line["decode"]["cold"] = {
            "ms_per_step": round(cold["cold_ms"], 5), "steps_per_s": round(1e3 / cold["cold_ms"], 1),
            "frac": round(cach / HBM_PEAK_GBS, 4), "achieved": round(cach, 1),
            "note": f"{cold['n']} x ({FLUSH_BYTES >> 20} MB scratch read, step) back to back "
                    f"minus {cold['n']} reads alone ({cold['fill_ms']:.4f} ms each), per step: "
                    "each step reads the state and its inputs from HBM, not the Infinity Cache"}
        b16 = rec.pop("bf16_state")
        step16 = b16["ms"] / S
        bytes16 = DECODE_STATE_BYTES // 2 + DECODE_TOKEN_BYTES
        ach16 = bytes16 / (step16 / 1e3) / 1e9
        line["decode_bf16_state"] = {
            "workload": "decode-64x256 as above with the state held in bf16 (fp32 arithmetic, "
                        "state rounded once per step when written)",
            "steps_per_s": round(1e3 / step16, 1), "ms_per_step": round(step16, 5),
            "eager_ms_per_step": b16["eager_ms_per_step"],
            "tokens_per_s": round(64 * 1e3 / step16, 1),
            "roofline": {"bound": "hbm", "achieved": round(ach16, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(ach16 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_bf16_state"),
                         "scope": f"bf16 state read + write once and the step's inputs and "
                                  f"outputs, {bytes16} bytes per step"},
        }
        line["recurrent_prefill"] = rec
    if not args.no_conv:
        log("causal conv leg")
        line["causal_conv"] = bench_conv(args, torch, kda)
    # CPU baselines last: the oracle's OpenMP threads must not compete with
    # the host thread that issues the GPU legs
    if not args.no_decode and not args.no_cpu:
        log("timing the CPU oracle (decode)")
        line["decode"]["cpu_baseline"] = cpu_decode_baseline(dinp, dec, dstate0)
    if not args.no_decode:
        del dec
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = 2 * n * 4
    if not args.no_cpu:
        log("timing the CPU oracle (prefill)")
        line["cpu_baseline"] = cpu_prefill_baseline(args, inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
