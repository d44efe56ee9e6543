#!/usr/bin/env python3
"""Decode throughput of the PACE periodic int4 state path on one MI355X.

Workload (PACE-4 decode): B = 64 sequences, 32 value heads over 16 key heads, d = 128,
bf16 q/k/v/o, symmetric int4 state with 64-key channel-aligned groups and bf16 scales,
int8 decode buffer, dP = 8, a 512-token context, L = 24 independent gated-delta layers
(the per-step working set, ~505 MB of state + buffer, is twice the 256 MB Infinity
Cache, so the state stream comes from HBM).  Inputs are seeded synthetic tensors with
the column-outlier structure (4 of 128 value channels per head scaled x8 on runs of
50-200 tokens), generated on the device; the 512-token context is written by
pace_prefill_chunk before timing.

One bench "step" = one decode period: dP tokens x L layers of pace_decode_step, i.e. every
decode row of the path (append, dequantise, replay, output, fold, requantise) once per
(layer, head, sequence).  A period is captured once in a HIP graph; `--warmup` replays are
untimed, then `--steps` replays are timed between two events on the launch stream with a
device synchronisation on both sides.  value = B * dP * steps / time.

roofline: the decode kernel's algorithmic bytes per launch (state read 8704 B, buffered
tokens read, q/k/v/a/beta in, append write, o out, and on flushing steps the 8704 B state
write, per (sequence, head)), averaged over the dP positions of a period, divided by the
mean launch duration in the timed region (timed-region time / launches; the graph holds
only decode launches).  traffic: HBM bytes per launch from rocprofv3 FETCH_SIZE +
WRITE_SIZE, scaled by the same counters on a copy of known size, read from the committed
counter summary when it was taken on the current kernel source, else null.
Also reported: same-box bounds for a launch of this shape (a no-op kernel and a read-only
stream of the same bytes in the same grid, timed in the same graph arrangement), the bf16
per-token-state baseline on the same tokens, PACE-4/8 with both buffers and the decode
buffer on a bf16 state at the same batch (with the split of the gain over the per-token
baseline into the buffer's share and the 4-bit state's share), a batch sweep
B = 1, 16, 32, 64, 128 (PACE-4, bf16 per-token and bf16-state periodic at each), the long
chunked prefill, and cpu_baseline: the fp64 oracle on a bounded sample of the same
workload on one host core.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--heads", type=int, default=32)
    ap.add_argument("--kv-heads", type=int, default=16)
    ap.add_argument("--dim", type=int, default=128)
    ap.add_argument("--dP", type=int, default=8)
    ap.add_argument("--context", type=int, default=512)
    ap.add_argument("--variant", choices=["pace4", "pace48-int8", "pace48-mixed", "bf16-periodic"], default="pace4")
    ap.add_argument("--variants", action="store_true", default=True,
                    help="also time PACE-4/8 (int8 and mixed buffers) and the bf16-state periodic decode")
    ap.add_argument("--no-variants", dest="variants", action="store_false")
    ap.add_argument("--ceilings", action="store_true", default=True)
    ap.add_argument("--no-ceilings", dest="ceilings", action="store_false")
    ap.add_argument("--baseline", action="store_true", default=True)
    ap.add_argument("--no-baseline", dest="baseline", action="store_false")
    ap.add_argument("--cpu-baseline", action="store_true", default=True)
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--staggered", action="store_true", default=True)
    ap.add_argument("--no-staggered", dest="staggered", action="store_false")
    ap.add_argument("--sweep", action="store_true", default=True)
    ap.add_argument("--no-sweep", dest="sweep", action="store_false")
    ap.add_argument("--sweep-batches", default="1,16,32,64,128")
    ap.add_argument("--prefill", action="store_true", default=True)
    ap.add_argument("--no-prefill", dest="prefill", action="store_false")
    ap.add_argument("--prefill-tokens", type=int, default=32768)
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--prefill-warmup", type=int, default=8)
    # profile post-processing (no GPU work): summaries of rocprofv3 CSV output
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT"))
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_LOG", "OUT_PREFIX"),
                    help="per decode layout: HBM bytes per launch from a FETCH_SIZE and a WRITE_SIZE run of "
                         "bench.py, against the algorithmic bytes in that run's JSON line (BENCH_LOG); writes "
                         "OUT_PREFIX<layout>_b<B>.txt")
    ap.add_argument("--launch-profile", action="store_true",
                    help="no timing: one layer of the configured layout, a prefilled context, then 2 x dP eager "
                         "decode launches (every position of the period twice), for a per-dispatch counter run")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("PMC_DIR", "OUT"),
                    help="per position of the period: SQ instruction counts per wave of the decode launches of a "
                         "--launch-profile counter run")
    ap.add_argument("--profile-command", default=None, help="command line(s) recorded in the summary")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ inputs ----

def make_layer_inputs(torch, B, T, Hv, Hk, d, seed, t_offset=0, timeline=768):
    """Seeded synthetic token inputs on the device (same distributions as the
    pace_synth generator: normalised q/k, N(0,1) v with column outliers,
    a = exp(-softplus(N(-4,1))), beta = sigmoid(N(0,1)))."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dev = "cuda"
    q = torch.randn((B, T, Hk, d), generator=g, device=dev)
    k = torch.randn((B, T, Hk, d), generator=g, device=dev)
    v = torch.randn((B, T, Hv, d), generator=g, device=dev)
    a = torch.exp(-torch.nn.functional.softplus(torch.randn((B, T, Hv), generator=g, device=dev) - 4.0))
    beta = torch.sigmoid(torch.randn((B, T, Hv), generator=g, device=dev))
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    # column outliers on the token timeline
    rng = np.random.default_rng(seed)
    chans = np.stack([rng.choice(d, size=4, replace=False) for _ in range(Hv)])        # [Hv, 4]
    on = np.zeros((B, Hv, 4, timeline), dtype=bool)
    for b in range(B):
        for h in range(Hv):
            for c in range(4):
                state = bool(rng.integers(0, 2))
                t = 0
                while t < timeline:
                    run = int(rng.integers(50, 201))
                    if state:
                        on[b, h, c, t:t + run] = True
                    state = not state
                    t += run
    on = torch.from_numpy(on[..., t_offset:t_offset + T]).to(dev)                      # [B, Hv, 4, T]
    gain = torch.where(on, 8.0, 1.0).permute(0, 3, 1, 2)                                # [B, T, Hv, 4]
    idx = torch.from_numpy(chans).to(dev).view(1, 1, Hv, 4).expand(B, T, Hv, 4)
    v.scatter_(3, idx, torch.gather(v, 3, idx) * gain)
    bf = torch.bfloat16
    return (q.to(bf).contiguous(), k.to(bf).contiguous(), v.to(bf).contiguous(),
            a.float().contiguous(), beta.float().contiguous())


# ------------------------------------------------------------------ timing ----

def algorithmic_bytes_per_launch(cfg, n0, L):
    """Bytes one pace_decode_step launch must move, per its definition, summed over the
    B x Hv tiles, for a buffer count n0 before the step.  State read, previous buffered
    tokens (k codes+scale per key head shared by gamma heads, v codes+scale, a, beta),
    current q/k/v (bf16) and a/beta, the appended token, o, and the state write on the
    flushing step."""
    B, Hv, Hk, d, dP = cfg.B, cfg.Hv, cfg.Hk, cfg.dk, cfg.dP
    gamma = Hv // Hk
    rec = L["seq_stride"] / Hv                            # mean record bytes per head
    if cfg.buf == "int8":
        tok = d / gamma + 4 / gamma + d + 4 + 4 + 4          # per value head: k(shared) + v + a + beta
    else:
        tok = d / 2 / gamma + 4 / gamma + 2 * d + 4 + 4
    io_in = (2 * d * 2) / gamma + d * 2 + 8                 # q, k (shared per key head), v, a, beta
    o_out = d * 2
    flush = (n0 + 1) >= dP
    per_tile = rec + n0 * tok + io_in + o_out + (rec if flush else tok)
    return per_tile * B * Hv


def kernel_durations(torch, stream, calls, periods=2):
    """Mean GPU duration of each launch in `calls`, from event pairs recorded around it on
    its stream, launched eagerly.  Every launch is enqueued behind a GPU spin first, so
    the brackets hold GPU work only; an event pair adds its own overhead, so these
    durations are an upper bound, used for the per-position (flush / no flush) split.
    Returns [periods, len(calls)] in ms."""
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(periods)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(2.4e9 * 0.2))          # ~0.2 s spin while the launches queue up
        for p in range(periods):
            for i, c in enumerate(calls):
                ev[p][i][0].record(stream)
                c()
                ev[p][i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([[s.elapsed_time(e) for s, e in row] for row in ev])


def time_graph(torch, stream, calls, steps, warmup, replay_ms=None):
    """Capture `calls` once in a HIP graph on `stream`; replay it `warmup` times untimed,
    then `steps` times between two events on that stream, with a device synchronisation
    on both sides.  Returns the timed milliseconds.  With a list `replay_ms`, `steps`
    further replays follow, each between its own pair of events, and their durations are
    appended to it (for the median per replay; not part of the returned time)."""
    with torch.cuda.stream(stream):
        for c in calls:                      # warm the path once outside capture
            c()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in calls:
            c()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    if replay_ms is not None:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        with torch.cuda.stream(stream):
            for e0, e1 in ev:
                e0.record(stream)
                graph.replay()
                e1.record(stream)
        torch.cuda.synchronize()
        replay_ms.extend(e0.elapsed_time(e1) for e0, e1 in ev)
    del graph
    return ms


def copy_ceiling(torch, nbytes=1 << 30, reps=5):
    """Device-to-device copy of `nbytes` (torch's vectorised copy kernel): the same-box
    streaming ceiling, counting read + write bytes."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (s.elapsed_time(e) / 1e3) / 1e9
    del src, dst
    return gbs


def measure_ceilings(torch, bytes_per_launch, gx, gy, layers, dP, steps, warmup, threads=128):
    """Same-box bounds for one decode launch of this shape, timed exactly like the decode (a
    graph of layers x dP launches on one stream, `warmup` untimed replays, then `steps`
    timed ones):
      empty  -- a kernel that does nothing, grid (gx, gy) x threads: the fixed cost of a
                launch of this shape in a graph (dispatch, start-up, end of kernel);
      stream -- a read-only non-temporal stream of the decode launch's byte count in the
                same grid, each layer on its own buffer (so, like the decode's states, the
                stream comes from HBM): the fastest a launch moving those bytes can be.
    Kernels from libpace_measure.so (include/pace_measure.h)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "bit_recurrent_state_amd", "libpace_measure.so"))
    lib.pace_measure_empty.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.pace_measure_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    wgs = gx * gy
    bpw = -(-int(bytes_per_launch) // (wgs * 16)) * 16
    bufs = [torch.zeros(bpw * wgs, dtype=torch.uint8, device="cuda") for _ in range(layers)]
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def checked(fn, *a):
        def call():
            r = fn(*a)
            if r != 0:
                raise RuntimeError(f"{fn.__name__} returned {r}")
        return call
    empty = [checked(lib.pace_measure_empty, gx, gy, threads, sp) for _ in range(layers * dP)]
    streams = [checked(lib.pace_measure_stream, ctypes.c_void_p(bufs[l].data_ptr()), bpw, gx, gy, threads,
                       ctypes.c_void_p(sink.data_ptr()), sp) for _ in range(dP) for l in range(layers)]
    ms_e = time_graph(torch, stream, empty, steps, warmup)
    ms_s = time_graph(torch, stream, streams, steps, warmup)
    n = layers * dP * steps
    e_us, s_us = ms_e * 1e3 / n, ms_s * 1e3 / n
    res = {"empty_launch_us": round(e_us, 3), "stream_launch_us": round(s_us, 3),
           "stream_bytes_per_launch": bpw * wgs, "stream_GBps": round(bpw * wgs / (s_us * 1e-6) / 1e9, 1),
           "shape": f"grid ({gx}, {gy}) x {threads} threads, {layers} buffers x {dP} launches per graph replay"}
    del bufs, sink
    torch.cuda.empty_cache()
    return res


def head_map(torch, pace, args, layer):
    """PACE-4/8 head map of one layer: e_h, a_h from a seeded 512-token calibration run on
    the GPU (pace_calibrate_heads, asymmetric 4-bit quantiser with 32-key groups), then the
    quarter of heads with the largest E_h at 8 bits (pace_head_alloc)."""
    d, Hv, Hk, dP = args.dim, args.heads, args.kv_heads, args.dP
    Bc = 2
    ccfg = pace.LayerConfig(B=Bc, Hv=Hv, Hk=Hk, dk=d, dv=d, group=32, asym=True, buf="int8",
                            bf16_io=True, dP=dP)
    q, k, v, a, beta = make_layer_inputs(torch, Bc, 512, Hv, Hk, d, 100000 + 1000 * (args.seed + 101) + layer,
                                         timeline=512)
    e_h, a_h = pace.calibrate_heads(ccfg, k, v, a, beta)
    bits, _ = pace.head_alloc(e_h.cpu().numpy(), a_h.cpu().numpy(), dP, int(Hv / 4 + 0.5))
    return [int(x) for x in bits]


def make_cfgs(torch, pace, args, B, variant=None):
    """One layer configuration per layer (PACE-4/8 layers differ in their head maps)."""
    d, Hv, Hk, dP = args.dim, args.heads, args.kv_heads, args.dP
    variant = variant or args.variant
    if variant == "pace4":
        return [pace.pace4(B=B, Hv=Hv, Hk=Hk, d=d, dP=dP)] * args.layers
    if variant == "bf16-periodic":
        return [pace.bf16_periodic(B=B, Hv=Hv, Hk=Hk, d=d, dP=dP)] * args.layers
    buf = "int8" if variant == "pace48-int8" else "mixed"
    return [pace.pace48(head_map(torch, pace, args, l), B=B, Hv=Hv, Hk=Hk, d=d, dP=dP, buf=buf)
            for l in range(args.layers)]


def build_layers(torch, pace, args, cfgs):
    """Per layer: a zeroed state and buffer, the context written by pace_prefill_chunk,
    and dP decode tokens."""
    layers = []
    for l in range(args.layers):
        cfg = cfgs[l]
        B, Hv, Hk, d, dP = cfg.B, cfg.Hv, cfg.Hk, cfg.dk, cfg.dP
        L = pace.layout(cfg)
        st = torch.zeros(L["state_bytes"], dtype=torch.uint8, device="cuda")
        bu = torch.zeros(L["buffer_bytes"], dtype=torch.uint8, device="cuda")
        ctx = make_layer_inputs(torch, B, args.context + dP, Hv, Hk, d, 1000 * args.seed + l)
        o = torch.empty((B, Hv, d), dtype=torch.bfloat16, device="cuda")
        if cfg.bf16_state:
            # a bf16 state takes no prefill call: the context is written token by token by
            # the per-token bf16 kernel, whose state layout it shares
            sb = st.view(torch.bfloat16)
            for t in range(args.context):
                pace.bf16_decode_step(cfg, sb, *(x[:, t].contiguous() for x in ctx), o)
        else:
            o_ctx = torch.empty((B, args.context, Hv, d), dtype=torch.bfloat16, device="cuda")
            pq, pk_, pv, pa, pb = (x[:, :args.context].contiguous() for x in ctx)
            ws_n = pace.prefill_workspace_bytes(cfg, args.context)
            ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda") if ws_n else None
            pace.prefill_chunk(cfg, st, pq, pk_, pv, pa, pb, o_ctx, workspace=ws)
            del o_ctx, pq, pk_, pv, pa, pb, ws
        toks = [tuple(x[:, args.context + t].contiguous() for x in ctx) for t in range(dP)]
        layers.append(dict(cfg=cfg, state=st, buf=bu, toks=toks, o=o))
        del ctx
    torch.cuda.synchronize()
    return layers, L


def run_decode(torch, pace, args, B, steps, warmup, split=False, phases=None, ordered=False, variant=None):
    """Decode periods of the L-layer stack at batch B.  Returns a dict of figures.

    phases: optional per-sequence buffer counts to start from (continuous batching:
    sequences that joined at different times flush at different steps).  They are set
    by decode steps under the active mask before timing; every sequence still passes
    through each count once per period, so the bytes and tokens of a period are those
    of the aligned case.  ordered: issue each step through pace_decode_step_ordered with
    the sequences that flush at that step placed first (what a continuous-batching
    scheduler, which knows every sequence's position in its period, would pass)."""
    t0 = time.time()
    cfgs = make_cfgs(torch, pace, args, B, variant)
    cfg = cfgs[0]
    dP, Lyr = cfg.dP, args.layers
    layers, L = build_layers(torch, pace, args, cfgs)
    if phases is not None:
        ph = np.asarray(phases)
        for k in range(1, dP):
            mask = torch.from_numpy((ph >= k).astype(np.uint8)).cuda()
            for ly in layers:
                q, k_, v, a, b_ = ly["toks"][k - 1]
                pace.decode_step(ly["cfg"], ly["state"], ly["buf"], q, k_, v, a, b_, ly["o"], active=mask)
        torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    calls = []
    for t in range(dP):
        order = None
        if ordered and phases is not None:
            flushing = (np.asarray(phases) + t) % dP == dP - 1
            order = np.concatenate([np.flatnonzero(flushing), np.flatnonzero(~flushing)])
        for ly in layers:
            q, k, v, a, b_ = ly["toks"][t]
            calls.append(pace.prepare_decode_step(ly["cfg"], ly["state"], ly["buf"], q, k, v, a, b_, ly["o"],
                                                  stream=stream, order=order))
    replays = []
    ms = time_graph(torch, stream, calls, steps, warmup, replay_ms=replays)
    n_launch = len(calls) * steps
    launch_s = ms / 1e3 / n_launch                       # mean launch duration in the timed region
    per_pos = np.array([algorithmic_bytes_per_launch(cfg, t, L) for t in range(dP)])
    bytes_per_launch = float(per_pos.mean())
    res = dict(cfg=cfg, L=L, B=B, ms=ms, ms_per_step=ms / steps, ms_per_step_median=float(np.median(replays)),
               tokens_per_s=B * dP * steps / (ms / 1e3),
               bytes_per_launch=bytes_per_launch, launch_us=launch_s * 1e6,
               achieved=bytes_per_launch / launch_s / 1e9,
               setup_s=time.time() - t0)
    if split:
        kern = kernel_durations(torch, stream, calls, periods=2).mean(axis=0).reshape(dP, Lyr)
        res["eager_us"] = float(kern.mean() * 1e3)
        res["eager_flush_us"] = float(kern[-1].mean() * 1e3)
        res["eager_noflush_us"] = float(kern[:-1].mean() * 1e3)
    res["layers"] = layers
    return res


MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}     # MI355X dense matrix peaks


def prefill_flops(T, Hv, B, d, bf16_io=True, chunk=256, sb=64):
    """Algorithmic and executed flops of pace_prefill_chunk over B x Hv (sequence, head)
    pairs of T tokens.  Algorithmic: the WY form on whole 256-token chunks (72.7 MFLOP per
    chunk-head at d = 128, triangular products counted once).  Executed: what the
    64-token sub-block kernel issues per workgroup and sub-block, by MFMA type -- with bf16
    inputs, bf16 16x16x32 MFMAs for K K^T and Q K^T (one pass) and for K S, Q S and the
    state update (three passes each: the fp32 operand as three bf16 pieces), and fp32
    16x16x4 MFMAs for the blocked solve and P U; with fp32 inputs, all fp32 16x16x4.
    At d >= 128 the library splits each pair over two column-block workgroups (always with
    bf16 inputs; with fp32 inputs when twice the pairs fit the 256 CUs of MI355X), which
    both issue the key-side products (K K^T, Q K^T)."""
    cs = 2 if (d >= 128 and (bf16_io or 2 * B * Hv <= 256)) else 1
    C = chunk
    per_chunk = 2 * (2.5 * C * C * d + 3 * C * d * d + C ** 3 / 6)
    alg = per_chunk * (-(-T // C)) * B * Hv
    tt, kt, ct = sb // 16, d // 16, d // 16          # token, key and column tiles
    pairs = tt * (tt + 1) // 2
    solve_f32 = (sum(4 * ib for ib in range(tt)) + 4 * tt) * ct
    pu_f32 = pairs * 4 * ct
    if bf16_io:
        bf16 = cs * 2 * pairs * (d // 32) + 2 * 3 * (kt // 2) * tt * ct + 3 * (tt // 2) * kt * ct
        f32 = solve_f32 + pu_f32
    else:
        bf16 = 0
        f32 = cs * 2 * pairs * (d // 4) + 2 * tt * kt * 4 * ct + solve_f32 + pu_f32 + tt * 4 * kt * ct
    n = -(-T // sb) * B * Hv
    return alg, {"bf16": bf16 * 2 * 16 * 16 * 32 * n, "f32": f32 * 2 * 16 * 16 * 4 * n}


def run_long_prefill(torch, pace, args):
    """Long chunked prefill: B = 4 sequences x 32,768 tokens, 32 value / 16 key heads,
    d = 128, bf16 q/k/v, fp32 gates, int4 g = 64 rounded once per 256-token chunk; then
    decode steps of that layer at dP = 8 (B = 4 under-fills the chip; reported only)."""
    B, T, Hv, Hk, d = 4, args.prefill_tokens, args.heads, args.kv_heads, args.dim
    cfg = pace.pace4(B=B, Hv=Hv, Hk=Hk, d=d, dP=args.dP)
    L = pace.layout(cfg)
    q, k, v, a, beta = make_layer_inputs(torch, B, T + 8 * args.dP, Hv, Hk, d, 4000 + args.seed, timeline=T + 8 * args.dP)
    pq, pk_, pv, pa, pb = (x[:, :T].contiguous() for x in (q, k, v, a, beta))
    o = torch.empty((B, T, Hv, d), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(L["state_bytes"], dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    call = pace.prepare_prefill_chunk(cfg, st, pq, pk_, pv, pa, pb, o, stream=stream)
    # untimed warm-up launches first: the first few ~3 ms launches on a fresh box run
    # slower until the clocks have settled (about 20 ms of work)
    times = []
    for rep in range(args.prefill_warmup + args.prefill_reps):
        st.zero_()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        with torch.cuda.stream(stream):
            call()
        e.record(stream)
        torch.cuda.synchronize()
        if rep >= args.prefill_warmup:
            times.append(s.elapsed_time(e))
    ms = float(np.median(times))
    alg, exe = prefill_flops(T, Hv, B, d, bf16_io=True)
    sec = ms / 1e3
    util = {k: round(v / sec / 1e12 / MFMA_PEAK_TFLOPS[k], 4) for k, v in exe.items()}
    res = {"workload": f"long chunked prefill B={B} x {T} tokens, {Hv} value / {Hk} key heads, d={d}, bf16 io, "
                       f"int4 g=64 rounded per 256-token chunk",
           "ms": round(ms, 3), "warmup_launches": args.prefill_warmup,
           "timed_launches": args.prefill_reps, "tokens_per_s": round(B * T / sec, 1),
           "algorithmic_TFLOP": round(alg / 1e12, 4), "algorithmic_TFLOPs": round(alg / sec / 1e12, 2),
           "executed_TFLOP": {k: round(v / 1e12, 4) for k, v in exe.items()},
           "executed_TFLOPs": {k: round(v / sec / 1e12, 2) for k, v in exe.items()},
           "mfma_peak_TFLOPs": MFMA_PEAK_TFLOPS,
           "mfma_util_of_dtype_peak": util,
           "note": "bf16 figures count the three split passes of the fp32 operands (exact bf16 "
                   "inputs times the state / decayed U as three bf16 pieces)",
           "workgroups": B * Hv * (2 if d >= 128 else 1), "threads_per_workgroup": 512 if d >= 128 else 256}
    log(f"long prefill: {ms:.2f} ms, {res['tokens_per_s']:,.0f} tok/s, executed "
        f"bf16 {res['executed_TFLOPs']['bf16']} TFLOP/s ({util['bf16']:.3f} of peak), "
        f"f32 {res['executed_TFLOPs']['f32']} TFLOP/s ({util['f32']:.3f} of peak), "
        f"algorithmic {res['algorithmic_TFLOPs']} TFLOP/s")
    # decode after the prompt: B = 4, one layer
    bu = torch.zeros(L["buffer_bytes"], dtype=torch.uint8, device="cuda")
    od = torch.empty((B, Hv, d), dtype=torch.bfloat16, device="cuda")
    toks = [tuple(x[:, T + t].contiguous() for x in (q, k, v, a, beta)) for t in range(8 * args.dP)]
    calls = [pace.prepare_decode_step(cfg, st, bu, *tk, od, stream=stream) for tk in toks]
    dms = time_graph(torch, stream, calls, max(2, args.steps // 4), 1)
    n = len(calls) * max(2, args.steps // 4)
    res["decode_after_prefill"] = {"B": B, "layers": 1, "tokens_per_s_per_layer": round(B * n / (dms / 1e3), 1),
                                   "mean_launch_us": round(dms * 1e3 / n, 3)}
    del q, k, v, a, beta, pq, pk_, pv, pa, pb, o, st, bu
    torch.cuda.empty_cache()
    return res


def decode_traffic(cfg_name):
    """HBM traffic per launch of the decode kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source (sha256 recorded with it)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_traffic_{cfg_name}.txt")
    src = os.path.join(ROOT, "bit_recurrent_state_amd", "csrc", "pace_decode.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != sha:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------- profile summaries ----

def _csv_rows(root, suffix):
    """Rows (dicts) of every rocprofv3 CSV under `root` whose name ends with `suffix`."""
    import csv
    rows = []
    for dp, _, files in os.walk(root):
        for f in sorted(files):
            if f.endswith(suffix):
                with open(os.path.join(dp, f), newline="") as fh:
                    rows.extend(csv.DictReader(fh))
    return rows


def _short(name, n=96):
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= n else name[:n - 3] + "..."


def summarize_trace(trace_dir, command):
    """Per-kernel duration statistics (microseconds) of a rocprofv3 --kernel-trace run."""
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    by = {}
    for r in rows:
        grid = "x".join(str(r.get(f"Grid_Size_{a}", r.get("Grid_Size", "?"))) for a in "XY")
        key = (r["Kernel_Name"], grid)
        by.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"command: {command}", "",
             f"{'kernel':98s} {'grid (threads)':>16s} {'calls':>7s} {'avg us':>9s} {'median':>9s} {'min':>9s} "
             f"{'max':>9s} {'total ms':>9s}"]
    for (name, grid), d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(d)
        lines.append(f"{_short(name):98s} {grid:>16s} {len(a):7d} {a.mean():9.3f} {np.median(a):9.3f} "
                     f"{a.min():9.3f} {a.max():9.3f} {a.sum() / 1e3:9.3f}")
    return "\n".join(lines)


def _counter_means(pmc_dir, counter):
    """{kernel name: (mean, min, max, dispatches)} of one counter (KiB per dispatch)."""
    rows = _csv_rows(pmc_dir, "counter_collection.csv")
    by = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (float(np.mean(v)), float(np.min(v)), float(np.max(v)), len(v)) for k, v in by.items()}


DECODE_LAYOUTS = {  # (buffer, head bits, bf16 state) of decode_kernel<D, TOK, BUF, HB, IO, GT, AS, NTS, ORD, BFS>
    "pace4": ("0", "4", "false"), "pace48-int8": ("0", "0", "false"), "pace48-mixed": ("1", "0", "false"),
    "bf16-periodic": ("0", "4", "true")}


def decode_layout(kernel_name):
    """The decode layout a decode_kernel instantiation serves (launch order only), or None."""
    if "decode_kernel<" not in kernel_name:
        return None
    args = [a.strip() for a in kernel_name.split("decode_kernel<", 1)[1].split(">", 1)[0].split(",")]
    if len(args) < 10 or args[8] != "false":
        return None
    for name, (buf, hb, bfs) in DECODE_LAYOUTS.items():
        if (args[2], args[3], args[9]) == (buf, hb, bfs):
            return name
    return None


def summarize_traffic(fetch_dir, write_dir, bench_log, copy_bytes, source, commands):
    """HBM traffic per dispatch of each decode layout's kernel, from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by what the same counter reads on the
    largest runtime device copy of the run (copy_bytes read and written: the 1 GiB copy
    bench.py times).  Returns {layout: summary text}."""
    import hashlib
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    res = [json.loads(l) for l in open(bench_log) if l.startswith("{")][-1]
    B = res["config"]["global_batch"]
    algo = {"pace4": res["roofline"]["bytes_per_launch"]}
    for v, leg in res.get("variants", {}).items():
        algo[v] = leg["bytes_per_launch"]
    # the dispatch of the runtime's copy kernel that moved the most bytes (the 1 GiB copy)
    copy_f = max(((k, v) for k, v in fetch.items() if "copyBuffer" in k), key=lambda kv: kv[1][2])
    copy_w = max(((k, v) for k, v in write.items() if "copyBuffer" in k), key=lambda kv: kv[1][2])
    kib = copy_bytes / 1024
    ff, fw = kib / copy_f[1][2], kib / copy_w[1][2]
    sha = hashlib.sha256(open(source, "rb").read()).hexdigest()
    out = {}
    for layout, a_bytes in algo.items():
        dk_f = [(k, v) for k, v in fetch.items() if decode_layout(k) == layout]
        dk_w = [(k, v) for k, v in write.items() if decode_layout(k) == layout]
        if not dk_f or not dk_w:
            continue
        n_f, n_w = sum(v[3] for _, v in dk_f), sum(v[3] for _, v in dk_w)
        f_mean = sum(v[0] * v[3] for _, v in dk_f) / n_f
        w_mean = sum(v[0] * v[3] for _, v in dk_w) / n_w
        fb, wb = f_mean * 1024 * ff, w_mean * 1024 * fw
        out[f"{layout}_b{B}"] = "\n".join([
            f"layout: {layout}, B = {B}; kernel(s): " + "; ".join(sorted({_short(k, 120) for k, _ in dk_f})),
            f"command_fetch: {commands[0]}", f"command_write: {commands[1]}",
            f"copy_fetch_KiB: {copy_f[1][2]:.1f}   ({_short(copy_f[0], 60)}: {kib:.0f} KiB read -> factor {ff:.4f})",
            f"copy_write_KiB: {copy_w[1][2]:.1f}   ({kib:.0f} KiB written -> factor {fw:.4f})",
            f"decode_fetch_KiB_raw: {f_mean:.1f} (min {min(v[1] for _, v in dk_f):.1f}, "
            f"max {max(v[2] for _, v in dk_f):.1f}, {n_f} dispatches)",
            f"decode_write_KiB_raw: {w_mean:.1f} (min {min(v[1] for _, v in dk_w):.1f}, "
            f"max {max(v[2] for _, v in dk_w):.1f}, {n_w} dispatches)",
            f"fetch_bytes_per_launch: {fb:.0f}", f"write_bytes_per_launch: {wb:.0f}",
            f"traffic_bytes_per_launch: {fb + wb:.0f}", f"algorithmic_bytes_per_launch: {a_bytes:.0f}",
            f"traffic_over_algorithmic: {(fb + wb) / a_bytes:.4f}",
            f"kernel_source_sha256: {sha}"])
    return out


SQ_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU",
               "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY")


def summarize_sq(pmc_dir, dP, command):
    """Per position of the decode period (count before the step; the last one flushes):
    mean SQ counts per wave over the decode_kernel dispatches of a --launch-profile run,
    taken in dispatch order (dispatch i sits at position i mod dP)."""
    rows = _csv_rows(pmc_dir, "counter_collection.csv")
    by = {}
    for r in rows:
        if "decode_kernel" not in r["Kernel_Name"]:
            continue
        d = by.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    names = [c for c in SQ_COUNTERS if any(c in d for d in by.values())]
    pos = {}
    for i, k in enumerate(sorted(by)):
        d = by[k]
        w = d.get("SQ_WAVES", 0.0)
        if w > 0:
            pos.setdefault(i % dP, []).append([d.get(c, 0.0) / w for c in names])
    lines = [f"command: {command}", "",
             "per wave, mean over the dispatches at each position of the period (position dP - 1 flushes)",
             f"{'position':>8s} " + " ".join(f"{c:>20s}" for c in names)]
    for t in sorted(pos):
        m = np.mean(np.array(pos[t]), axis=0)
        lines.append(f"{t:8d} " + " ".join(f"{x:20.1f}" for x in m))
    return "\n".join(lines)


def launch_profile(torch, pace, args):
    """One layer of the configured layout at batch args.batch: the context written by
    pace_prefill_chunk, then 2 x dP eager decode launches (no timing)."""
    cfg = make_cfgs(torch, pace, args, args.batch, None)[0]
    B, Hv, Hk, d, dP = cfg.B, cfg.Hv, cfg.Hk, cfg.dk, cfg.dP
    L = pace.layout(cfg)
    st = torch.zeros(L["state_bytes"], dtype=torch.uint8, device="cuda")
    bu = torch.zeros(L["buffer_bytes"], dtype=torch.uint8, device="cuda")
    x = make_layer_inputs(torch, B, args.context + 2 * dP, Hv, Hk, d, 1000 * args.seed)
    o = torch.empty((B, Hv, d), dtype=torch.bfloat16, device="cuda")
    if cfg.bf16_state:           # (no prefill call for a bf16 state: the per-token kernel writes it)
        for t in range(args.context):
            pace.bf16_decode_step(cfg, st.view(torch.bfloat16), *(y[:, t].contiguous() for y in x), o)
    else:
        o_ctx = torch.empty((B, args.context, Hv, d), dtype=torch.bfloat16, device="cuda")
        pace.prefill_chunk(cfg, st, *(t[:, :args.context].contiguous() for t in x), o_ctx)
        del o_ctx
    toks = [tuple(t[:, args.context + i].contiguous() for t in x) for i in range(2 * dP)]
    torch.cuda.synchronize()
    for tk in toks:
        pace.decode_step(cfg, st, bu, *tk, o)
    torch.cuda.synchronize()
    log(f"launch profile: {2 * dP} decode launches of one {args.variant} layer at B={B}")


def main():
    args = parse()
    if args.summarize_trace:
        d, out = args.summarize_trace
        open(out, "w").write(summarize_trace(d, args.profile_command or "") + "\n")
        return
    if args.summarize_traffic:
        fd, wd, blog, prefix = args.summarize_traffic
        cmds = (args.profile_command or " | ").split(" | ")
        txt = summarize_traffic(fd, wd, blog, 1 << 30,
                                os.path.join(ROOT, "bit_recurrent_state_amd", "csrc", "pace_decode.hip"), cmds)
        for name, body in txt.items():
            open(f"{prefix}{name}.txt", "w").write(body + "\n")
        return
    if args.summarize_sq:
        d, out = args.summarize_sq
        open(out, "w").write(summarize_sq(d, args.dP, args.profile_command or "") + "\n")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the PACE decode path here runs on a single MI355X "
              f"and has no multi-GPU mode (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_recurrent_state_amd as pace

    torch.cuda.set_device(0)
    if args.launch_profile:
        launch_profile(torch, pace, args)
        return
    B, Hv, Hk, d, dP, Lyr = args.batch, args.heads, args.kv_heads, args.dim, args.dP, args.layers
    if args.variant == "pace4":
        cfg0 = pace.pace4(B=B, Hv=Hv, Hk=Hk, d=d, dP=dP)
    elif args.variant == "bf16-periodic":
        cfg0 = pace.bf16_periodic(B=B, Hv=Hv, Hk=Hk, d=d, dP=dP)
    else:
        cfg0 = pace.pace48([8] * (Hv // 4) + [4] * (Hv - Hv // 4), B=B, Hv=Hv, Hk=Hk, d=d, dP=dP,
                           buf="int8" if args.variant == "pace48-int8" else "mixed")
    L0 = pace.layout(cfg0)
    log(f"variant {args.variant} B={B} Hv={Hv} Hk={Hk} d={d} dP={dP} layers={Lyr} "
        f"state/layer {L0['state_bytes'] / 1e6:.1f} MB buffer/layer {L0['buffer_bytes'] / 1e6:.1f} MB")

    r = run_decode(torch, pace, args, B, args.steps, args.warmup, split=True)
    log(f"decode: {r['tokens_per_s']:,.0f} tok/s, {r['ms_per_step']:.3f} ms/period, {r['launch_us']:.2f} us "
        f"per launch in the graph = {r['achieved']:.0f} GB/s; eager brackets: {r['eager_noflush_us']:.2f} us "
        f"without flush, {r['eager_flush_us']:.2f} us with (setup {r['setup_s']:.1f}s)")
    cfg, layers = r["cfg"], r.pop("layers")
    ceiling = copy_ceiling(torch)
    log(f"device copy (torch, 1 GiB) {ceiling:.0f} GB/s")
    ceil = None
    if args.ceilings:
        ceil = measure_ceilings(torch, r["bytes_per_launch"], Hv, B, Lyr, dP, args.steps, args.warmup)
        log(f"ceilings at this launch shape: {ceil}")
    traffic = decode_traffic(args.variant + f"_b{B}")

    result = {
        "metric": "decode tokens/s & achieved HBM GB/s (% peak), int4 state dP=8, B=1..128",
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "ms_per_step_median": round(r["ms_per_step_median"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"pace4": "int4 state / int8 buffer / bf16 io, fp32 + int32 accumulate",
                  "pace48-int8": "int4 + int8 (quarter of heads) state / int8 buffer / bf16 io, fp32 + int32 accumulate",
                  "pace48-mixed": "int4 + int8 (quarter of heads) state / 4-bit key + bf16 value buffer / bf16 io, "
                                  "fp32 + int32 accumulate",
                  "bf16-periodic": "bf16 state / int8 buffer / bf16 io, fp32 accumulate"}[args.variant],
        "data": "synthetic (seeded; column-outlier value channels)",
        "config": {"workload": f"{args.variant} decode, {Lyr} gated-delta layers x {Hv} value heads "
                               f"({Hk} key heads), d={d}, B={B}, dP={dP}, {args.context}-token context; "
                               f"step = one decode period ({dP} tokens x {Lyr} layers)",
                   "global_batch": B, "seq_len": args.context, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(r["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": "pace decode_kernel (pace_decode_step)",
                     "bytes_per_launch": round(r["bytes_per_launch"]),
                     "mean_launch_us": round(r["launch_us"], 3),
                     "eager_launch_us": {"no_flush": round(r["eager_noflush_us"], 3),
                                         "flush": round(r["eager_flush_us"], 3)},
                     "device_copy_GBps": round(ceiling, 1)},
    }
    if ceil is not None:
        result["roofline"].update({
            "stream_ceiling_GBps": ceil["stream_GBps"], "frac_of_stream_ceiling": round(r["achieved"] / ceil["stream_GBps"], 4),
            "empty_launch_us": ceil["empty_launch_us"], "stream_launch_us": ceil["stream_launch_us"],
            "ceiling_note": "stream: a read-only stream of the same bytes per launch in the decode's grid, timed in "
                            "the same graph arrangement; empty: a no-op kernel of that grid (libpace_measure.so)"})

    # ---- bf16 per-token-state baseline on the same shape
    if args.baseline:
        result["bf16_baseline"] = run_bf16_baseline(torch, pace, args, cfg, layers)
    del layers
    torch.cuda.empty_cache()

    # ---- the other decode layouts at the same batch: PACE-4/8 with both buffers (head maps
    # from the GPU calibration) and the decode buffer on a bf16 state
    if args.variants and args.variant == "pace4":
        legs = {}
        for v in ("pace48-int8", "pace48-mixed", "bf16-periodic"):
            rv = run_decode(torch, pace, args, B, args.steps, args.warmup, variant=v)
            legs[v] = {"tokens_per_s": round(rv["tokens_per_s"], 1), "ms_per_step": round(rv["ms_per_step"], 4),
                       "mean_launch_us": round(rv["launch_us"], 3), "bytes_per_launch": round(rv["bytes_per_launch"]),
                       "roofline": {"bound": "hbm", "achieved": round(rv["achieved"], 1), "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": round(rv["achieved"] / HBM_PEAK_GBS, 4)}}
            tv = decode_traffic(v + f"_b{B}")
            legs[v]["roofline"]["traffic"] = None if tv is None else round(tv)
            log(f"{v}: {legs[v]}")
            del rv["layers"]
            torch.cuda.empty_cache()
        result["variants"] = legs
        if args.baseline:
            bl, bp = result["bf16_baseline"]["value"], legs["bf16-periodic"]["tokens_per_s"]
            result["gain_split"] = {
                "note": "decode tokens/s at this batch: per-token bf16 state -> decode buffer on a bf16 state -> "
                        "decode buffer on the PACE-4 state ([p1] 'Assumptions and limits' attributes most of the gain "
                        "to the buffer)",
                "bf16_per_token": bl, "bf16_periodic": bp, "pace4": round(r["tokens_per_s"], 1),
                "buffer_share_x": round(bp / bl, 3), "int4_state_share_x": round(r["tokens_per_s"] / bp, 3),
                "total_x": round(r["tokens_per_s"] / bl, 3)}

    # ---- continuous batching: the same stack with every sequence at its own point of
    # the period (seeded uniform phases), so each step flushes about 1/dP of the tiles
    if args.staggered:
        phases = np.random.default_rng(args.seed + 17).integers(0, dP, size=B)
        stag = {"workload": "as config, each sequence starting at a seeded uniform random position of its "
                            f"{dP}-token period (flushes spread over the steps)"}
        for key, ordered in (("sequence_order", True), ("launch_order", False)):
            rs = run_decode(torch, pace, args, B, args.steps, args.warmup, phases=phases, ordered=ordered)
            stag[key] = {"tokens_per_s": round(rs["tokens_per_s"], 1), "ms_per_step": round(rs["ms_per_step"], 4),
                         "mean_launch_us": round(rs["launch_us"], 3), "GBps": round(rs["achieved"], 1),
                         "frac": round(rs["achieved"] / HBM_PEAK_GBS, 4),
                         "vs_aligned": round(rs["tokens_per_s"] / r["tokens_per_s"], 4)}
            del rs["layers"]
            torch.cuda.empty_cache()
        stag["note"] = ("sequence_order: pace_decode_step_ordered with the sequences that flush at each step "
                        "placed first; launch_order: pace_decode_step (sequence b on workgroup row b)")
        result["staggered_phases"] = stag
        log(f"staggered phases: {stag}")

    # ---- batch sweep (PACE-4 and the bf16 baseline at each B)
    if args.sweep:
        sweep = []
        for Bs in [int(x) for x in args.sweep_batches.split(",")]:
            rs = run_decode(torch, pace, args, Bs, max(3, args.steps // 2), args.warmup)
            ent = {"B": Bs, "tokens_per_s": round(rs["tokens_per_s"], 1), "GBps": round(rs["achieved"], 1),
                   "mean_launch_us": round(rs["launch_us"], 3),
                   "working_set_MB": round((rs["L"]["state_bytes"] + rs["L"]["buffer_bytes"]) * Lyr / 1e6, 1)}
            if args.ceilings and Bs > B:
                # the same-box streaming ceiling and launch floor at this batch's launch shape
                cb = measure_ceilings(torch, rs["bytes_per_launch"], Hv, Bs, Lyr, dP, max(3, args.steps // 2),
                                      args.warmup)
                ent.update({"stream_ceiling_GBps": cb["stream_GBps"], "stream_launch_us": cb["stream_launch_us"],
                            "empty_launch_us": cb["empty_launch_us"],
                            "frac_of_stream_ceiling": round(rs["achieved"] / cb["stream_GBps"], 4)})
            if args.baseline:
                bl = run_bf16_baseline(torch, pace, args, rs["cfg"], rs["layers"], steps=max(3, args.steps // 2),
                                       warmup=args.warmup, split=False)
                ent["bf16_tokens_per_s"] = bl["value"]
                ent["bf16_GBps"] = bl["timed_region_GBps"]
                ent["speedup_vs_bf16"] = round(rs["tokens_per_s"] / bl["value"], 3)
            del rs["layers"]
            torch.cuda.empty_cache()
            if args.variants and args.variant == "pace4":
                rp = run_decode(torch, pace, args, Bs, max(3, args.steps // 2), args.warmup, variant="bf16-periodic")
                ent["bf16_periodic_tokens_per_s"] = round(rp["tokens_per_s"], 1)
                ent["bf16_periodic_GBps"] = round(rp["achieved"], 1)
                del rp["layers"]
                torch.cuda.empty_cache()
            log(f"sweep B={Bs}: {ent}")
            sweep.append(ent)
        result["batch_sweep"] = sweep
    if args.prefill:
        result["long_prefill"] = run_long_prefill(torch, pace, args)
    torch.cuda.synchronize()
    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, Hv * Lyr)
    print(json.dumps(result), flush=True)


def run_bf16_baseline(torch, pace, args, cfg, layers, steps=None, warmup=None, split=True):
    """The bf16 per-token-state decode (pace_bf16_decode_step) over the same tokens:
    read S, update, write S every token."""
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    B, Hv, Hk, d, dP, Lyr = cfg.B, cfg.Hv, cfg.Hk, cfg.dk, cfg.dP, args.layers
    bcfg = pace.LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=cfg.group, bf16_io=True, dP=dP)
    states = [torch.randn((B, Hv, d, d), device="cuda").mul_(0.05).to(torch.bfloat16) for _ in range(Lyr)]
    stream = torch.cuda.Stream()
    calls = []
    for t in range(dP):
        for l, ly in enumerate(layers):
            q, k, v, a, b_ = ly["toks"][t]
            calls.append(pace.prepare_bf16_decode_step(bcfg, states[l], q, k, v, a, b_, ly["o"], stream=stream))
    ms = time_graph(torch, stream, calls, steps, warmup)
    tps = B * dP * steps / (ms / 1e3)
    per_launch = B * Hv * (2 * d * d * 2 + (2 * d * 2) / (Hv // Hk) + 2 * d * 2 + 8)
    launch_us = ms * 1e3 / (len(calls) * steps)
    gbs = per_launch / (launch_us / 1e6) / 1e9
    out = {"value": round(tps, 1), "unit": "tokens/s", "timed_region_GBps": round(gbs, 1),
           "bytes_per_launch": per_launch, "mean_launch_us": round(launch_us, 3)}
    msg = f"bf16 per-token baseline B={B}: {tps:,.0f} tok/s, {launch_us:.2f} us per launch = {gbs:.0f} GB/s"
    if split:
        kms = kernel_durations(torch, stream, calls, periods=1).mean()
        out["eager_launch_us"] = round(float(kms) * 1e3, 3)
        msg += f" (eager bracket {kms * 1e3:.2f} us)"
    log(msg)
    del states
    return out


def cpu_baseline(args, tiles_per_token):
    """fp64 oracle (as written, untuned) on a bounded sample of the same workload: the
    PACE-4 layer shape, a handful of (sequence, head) tiles, decode steps covering a
    flush, from a seeded random packed state.  Reported as decode tokens/s of the full
    stack, i.e. tile-steps/s divided by the tiles one token needs (heads x layers)."""
    from oracle import packing as pk
    from pace_synth import make_tokens, random_buffer_parts, random_packed_state_parts
    d, Hv, Hk, dP = args.dim, args.heads, args.kv_heads, args.dP
    Bs = 2
    ocfg = pk.LayerCfg(B=Bs, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, asym=False, buf="int8", dP=dP, bf16_io=True)
    st = pk.pack_state(ocfg, pk.state_from_parts(ocfg, random_packed_state_parts(5, Bs, Hv, d, d, 64, [4] * Hv, False)))
    bu = pk.pack_buffer(ocfg, random_buffer_parts(6, Bs, Hv, Hk, d, d, dP, False, counts=[0] * Bs))
    toks = make_tokens(7, Bs, 64, Hv, Hk, d, d, bf16=True)
    tiles = [(b, h) for b in range(Bs) for h in range(0, Hv, 4)]
    from threadpoolctl import threadpool_limits

    def rate(limit, seconds):
        """(tile-steps, seconds, decode steps) of the oracle with BLAS at `limit` threads."""
        nonlocal st, bu
        with threadpool_limits(limits=limit):
            t0 = time.time()
            steps = 0
            while True:
                o, st, bu, _ = pk.decode_step_layer(ocfg, st, bu, *toks.token(steps % 64), tiles=tiles)
                steps += 1
                if time.time() - t0 > seconds and steps % dP == 0:
                    break
            return steps * len(tiles), time.time() - t0, steps

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    # one host thread (the reported figure), then BLAS free to use every allowed core
    tile_steps, el, steps = rate(1, args.cpu_seconds / 2)
    ts_all, el_all, _ = rate(None, args.cpu_seconds / 2)
    threads = os.environ.get("OMP_NUM_THREADS", "unset")
    return {"value": round(tile_steps / el / tiles_per_token, 3), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{tile_steps} tile-steps ({len(tiles)} (seq, head) tiles x {steps} decode steps incl. "
                      f"{steps // dP} flushes) of the PACE-4 layer shape in {el:.1f}s, single-threaded "
                      f"Python/NumPy fp64 (BLAS limited to 1 thread); tokens/s = tile-steps/s / ({tiles_per_token} tiles per token); "
                      f"host affinity {cores} cores, OMP_NUM_THREADS={threads}",
            "all_cores": {"value": round(ts_all / el_all / tiles_per_token, 3), "unit": "tokens/s",
                          "blas_threads": cores,
                          "note": f"the same oracle and sample for {el_all:.1f}s with BLAS free to use all "
                                  f"{cores} allowed cores"},
            "tiny_reference": tiny_reference_time()}


def tiny_reference_time():
    """The oracle end to end on the tiny reference configuration (2 sequences, 4 heads,
    d = 64, fp32, symmetric int4 g = 32, int8 buffer, dP = 8): a 512-token prefill in two
    chunks, then 64 decode steps (8 flushes), one host thread."""
    from oracle import packing as pk
    from pace_synth import make_tokens
    from threadpoolctl import threadpool_limits
    ocfg = pk.LayerCfg(B=2, Hv=4, Hk=4, dk=64, dv=64, group=32, asym=False, buf="int8", dP=8, bf16_io=False)
    toks = make_tokens(0, 2, 576, 4, 4, 64, 64)
    tiles = [(b, h) for b in range(2) for h in range(4)]
    with threadpool_limits(limits=1):
        t0 = time.time()
        state = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
        for c in range(2):
            _, state, _ = pk.prefill_layer(ocfg, state, *toks.span(256 * c, 256 * (c + 1)), tiles=tiles)
        buffer = np.zeros(pk.buffer_layout(ocfg)[1], dtype=np.uint8)
        for t in range(512, 576):
            _, state, buffer, _ = pk.decode_step_layer(ocfg, state, buffer, *toks.token(t))
        el = time.time() - t0
    return {"seconds": round(el, 2), "workload": "tiny reference: B=2, 4 heads, d=64, fp32, sym int4 g=32, "
            "512-token prefill (2 chunks) + 64 decode tokens (8 flushes), oracle on one host thread",
            "tokens_per_s": round(2 * 576 / el, 1)}


if __name__ == "__main__":
    main()
