"""Benchmark: fused HC sublayer boundary, prefill T=4096, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode lag|fresh] [--no-cpu]

One step = one sublayer-boundary call over the whole 4096-token batch (the
prefill workload: B=1, T=4096, hc=4, d=5120, 20 Sinkhorn rounds, RMSNorm):
hc_post(delta, X, post, comb) -> hc_mixes on X' -> split/Sinkhorn -> hc_pre ->
RMSNorm.  --mode lag (the default) reads with the pre of the previous
boundary, the data flow of the pages' Block.forward: one kernel of libhc, X
read once, the workgroups of a token tile exchanging their per-slice sums on
chip.  --mode fresh reads X' with the pre this call derives: two kernels
(stream_kernel, then finish_kernel, which reads X' back).  Both modes are
timed and reported; --mode picks the headline.  Inputs are seeded synthetic tensors
(transformer_hyper_connection_amd.synth, workload "prefill"), resident in HBM
before timing; several input/output buffer sets rotate.  Prints one JSON line.

Beside the headline line: the decode block's glue (n=128, "decode"), the
same boundary at hc = 2 and 8 ("other_hc") and at n = 128 ... 32768
("sweep"), the calls at the stand-in stack's two ends ("stack_ends"), the
standalone entry points ("entry_points") and the given-pre call on its two
schedules, one launch and two ("schedules"), each timed by events.

Timing: after half a second of plain streaming (GPU clocks settle; the first
~20 ms after idle run several percent slower), W untimed warm-up steps; then
K steps timed by the host clock between two device synchronisations (value,
ms_per_step); then K more steps between two events on the launch stream (the
roofline: algorithmic bytes of a call / mean event time of a call); then, for
a two-kernel call, K more with events also between its two kernels (each
kernel's share; those events add a few microseconds per call).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import transformer_hyper_connection_amd as T  # noqa: E402
from transformer_hyper_connection_amd import profsum, synth  # noqa: E402

N_TOK = synth.WORKLOAD_TOKENS["prefill"]
HC, D, MIX = 4, 5120, 24
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_boundary_prefill_t4096.json")
# algorithmic bytes: per token  X 4*d*2 + delta d*2 + X' 4*d*2 + z d*2 (bf16)
#                               + post_in/comb_in 16+64 (+ pre_in 16 with a given pre) + pre/post/comb out 96
#                    per call   hc_fn (fp32) 24*4d*4 + base 96 + scale 12 + gamma d*4
BYTES_TOKEN_COMMON = 4 * D * 2 + D * 2 + 4 * D * 2 + D * 2 + 16 + 64 + 96
BYTES_CALL = MIX * 4 * D * 4 + MIX * 4 + 3 * 4 + D * 4
# the kernels of one call as rocprofv3 names them (the last template argument of
# exchange_kernel is whether the weight is stream-summed, the one before it
# the slice width in 64-feature chunks)
KERNELS = {"fresh": ("stream_kernel<2, true, false>", "finish_kernel<2, true>"),
           "lag": ("exchange_kernel<true, false, 20, false>",)}


def algorithmic_bytes(n: int, mode: str) -> int:
    per_tok = BYTES_TOKEN_COMMON + (16 if mode == "lag" else 0)
    return n * per_tok + BYTES_CALL


def bf(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def make_sets(s, dev, n_sets):
    base = {"x": bf(s["x"], dev), "delta": bf(s["delta"], dev), "post_in": f32(s["post_in"], dev),
            "comb_in": f32(s["comb_in"], dev), "pre_in": f32(s["pre_in"], dev)}
    sets = []
    for i in range(n_sets):
        ins = base if i == 0 else {k: v.clone() for k, v in base.items()}
        outs = {"x_out": torch.empty(N_TOK, HC, D, dtype=torch.bfloat16, device=dev),
                "y": torch.empty(N_TOK, D, dtype=torch.bfloat16, device=dev),
                "pre": torch.empty(N_TOK, HC, device=dev), "post": torch.empty(N_TOK, HC, device=dev),
                "comb": torch.empty(N_TOK, HC, HC, device=dev)}
        sets.append((ins, outs))
    return sets


def time_mode(mode, sets, params, steps, warmup):
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    calls = [T.BoundaryCall(ins["x"], delta=ins["delta"], post_in=ins["post_in"], comb_in=ins["comb_in"],
                            pre_in=ins["pre_in"] if mode == "lag" else None, out=outs, **params)
             for ins, outs in sets]
    for i in range(warmup):
        calls[i % len(calls)].run(sid)
    torch.cuda.synchronize()
    # the timed steps: host clock between two synchronisations
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % len(calls)].run(sid)
    host_enqueue = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same steps again between two events on the launch stream: the mean call
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        calls[i % len(calls)].run(sid)
    e1.record(stream)
    torch.cuda.synchronize()
    mean_call = e0.elapsed_time(e1) / steps
    out = {"wall_s": wall, "host_enqueue_us_per_call": host_enqueue / steps * 1e6, "mean_call_ms": mean_call}
    if len(KERNELS[mode]) == 1:
        return out
    # and once more with an event before, between and after the two kernels of
    # each call: their split (the events themselves add a few microseconds)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        c = calls[i % len(calls)]
        ev[i][0].record(stream)
        c.begin(sid)
        ev[i][1].record(stream)
        c.end(sid)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    k1 = [e[0].elapsed_time(e[1]) for e in ev]
    k2 = [e[1].elapsed_time(e[2]) for e in ev]
    call = [e[0].elapsed_time(e[2]) for e in ev]
    return {**out, "call_ms": call, "stream_kernel_ms": k1, "finish_kernel_ms": k2}


def settle_clocks(dev, seconds=0.5):
    """Keep the GPU streaming for a moment before anything is timed: the first
    ~20 ms of work after idle run several percent slower."""
    a = torch.empty(1 << 27, dtype=torch.bfloat16, device=dev).fill_(1)
    b = torch.empty_like(a)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            torch.mul(a, 1, out=b)
        torch.cuda.synchronize()
    del a, b


def reference_stream(dev, nbytes=1 << 30, reps=10):
    """A plain streaming kernel over 1 GiB (read 1 GiB, write 1 GiB, one dispatch):
    the practical HBM ceiling on this device, and the size reference for the
    traffic counters."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1, out=b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mul(a, 1, out=b)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def traffic(mode):
    """HBM bytes of one call from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != profsum.source_sha256():
        return None, "kernel source changed since the counters were taken"
    total = 0
    for want in KERNELS[mode]:
        hit = [v for k, v in t["kernels"].items() if want in k]
        if not hit:
            return None, f"{want} not in the counter summary"
        total += hit[0]["fetch_bytes"] + hit[0]["write_bytes"]
    return total, os.path.relpath(TRAFFIC_FILE, ROOT)


def cpu_baseline(s, repeats, mode):
    """The CPU oracle on the same workload (the headline read mode), timed on
    this host."""
    from oracle import hc_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        O.boundary(x=s["x"], delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"],
                   pre_in=s["pre_in"] if mode == "lag" else None,
                   hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"], gamma=s["gamma"])
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"value": round(N_TOK / med, 1), "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"the whole {N_TOK}-token prefill batch, {'given' if mode == 'lag' else 'fresh'}-pre "
                      f"boundary with the RMSNorm, median of "
                      f"{repeats} runs ({med:.2f} s each); float64 BLAS projection on {blas_threads} threads, "
                      f"fp32/fp64 elementwise NumPy on 1 thread; {len(os.sched_getaffinity(0))} usable host "
                      f"cores, os.cpu_count()={os.cpu_count()}"}


def decode_block(dev, reps=200):
    """The decode block's glue (B=128, T=1: the entry read with the incoming
    mix, the boundary, the last write; each read with its RMSNorm, as the
    pages' block normalises every sublayer input), eager and replayed from a
    captured graph; mean microseconds per block and per boundary call over
    reps, and the boundary call without the RMSNorm."""
    b = synth.block_inputs()
    (fa, ba, sa), (ff, bf_, sf) = b["attn"], b["ffn"]
    A = dict(fn_packed=T.hc_fn_pack(f32(fa, dev)), hc_base=f32(ba, dev), hc_scale=f32(sa, dev))
    F = dict(fn_packed=T.hc_fn_pack(f32(ff, dev)), hc_base=f32(bf_, dev), hc_scale=f32(sf, dev))
    X, PRE, DA, DF = bf(b["x"], dev), f32(b["pre_in"], dev), bf(b["delta_attn"], dev), bf(b["delta_ffn"], dev)
    g = f32(synth.gamma("decode", 90), dev)
    entry = T.BoundaryCall(X, pre_in=PRE, gamma=g, **A)
    e = entry.outputs
    bnd = T.BoundaryCall(X, delta=DA, post_in=e["post"], comb_in=e["comb"], pre_in=e["pre"], gamma=g, **F)
    bnd_plain = T.BoundaryCall(X, delta=DA, post_in=e["post"], comb_in=e["comb"], pre_in=e["pre"], **F)
    o = bnd.outputs
    xo = torch.empty_like(X)

    def glue():
        entry.run()
        bnd.run()
        T.hc_post(DF, o["x_out"], o["post"], o["comb"], out=xo)

    def timed(fn):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    eager = timed(glue)
    boundary = timed(bnd.run)
    boundary_plain = timed(bnd_plain.run)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        glue()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        glue()
    graph = timed(g.replay)
    return {"workload": "decode block glue, B=128 T=1, hc=4, d=5120: entry (incoming mix) + boundary "
                        "(attention pre) + last write; given pre, each read with its RMSNorm",
            "tokens": int(X.shape[0]), "block_us_eager": round(eager, 2), "block_us_graph": round(graph, 2),
            "boundary_call_us": round(boundary, 2), "boundary_call_us_no_rmsnorm": round(boundary_plain, 2)}


def decode_stack(dev, sublayers=80, reps=20):
    """A decode stack's glue (B=128, T=1): the entry (read with the incoming
    mix), then one boundary per sublayer (write with the previous post/comb,
    mixes, read with the previous pre, RMSNorm), the attention and
    feed-forward parameter sets alternating and a given stand-in sublayer
    output; eager (each call enqueued by the binding) and replayed from one
    captured graph.  Mean microseconds per sublayer."""
    b = synth.block_inputs()
    sets = [dict(fn_packed=T.hc_fn_pack(f32(fn, dev)), hc_base=f32(base, dev), hc_scale=f32(scale, dev))
            for fn, base, scale in (b["attn"], b["ffn"])]
    g = torch.ones(D, dtype=torch.float32, device=dev)
    X, PRE = bf(b["x"], dev), f32(b["pre_in"], dev)
    DL = bf(b["delta_attn"], dev)
    calls = [T.BoundaryCall(X, pre_in=PRE, gamma=g, **sets[0])]
    for i in range(sublayers):
        o = calls[-1].outputs
        x_in = X if i == 0 else o["x_out"]
        calls.append(T.BoundaryCall(x_in, delta=DL, post_in=o["post"], comb_in=o["comb"], pre_in=o["pre"], gamma=g,
                                    **sets[(i + 1) % 2]))

    def stack():
        for c in calls:
            c.run()

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3 / len(calls)

    eager = timed(stack)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stack()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack()
    replay = timed(graph.replay)
    return {"workload": f"decode stack glue, B=128 T=1, hc=4, d=5120: the entry and {sublayers} sublayer "
                        "boundaries (given pre, RMSNorm), eager and from one captured graph",
            "calls": len(calls), "per_call_us_eager": round(eager, 2), "per_call_us_graph": round(replay, 2)}


def other_hc(dev, hcs=(2, 8), reps=50):
    """The same boundary (write, fresh pre, RMSNorm; n=4096, d=5120) at hc = 2
    and 8, which libhc runs as four plainer launches (row write, matrix-core
    projection, finish, row read).  Mean microseconds per call by events over
    at least reps calls after a warm-up, and the algorithmic bytes of a call."""
    out = {}
    for hc in hcs:
        print(f"[bench] timing hc={hc}", file=sys.stderr, flush=True)
        s = synth.boundary_inputs("prefill", hc=hc)
        mix = (2 + hc) * hc
        call = T.BoundaryCall(bf(s["x"], dev), delta=bf(s["delta"], dev), post_in=f32(s["post_in"], dev),
                              comb_in=f32(s["comb_in"], dev), fn_packed=T.hc_fn_pack(f32(s["hc_fn"], dev), hc=hc),
                              hc_base=f32(s["hc_base"], dev), hc_scale=f32(s["hc_scale"], dev),
                              gamma=f32(s["gamma"], dev))
        us = timed_calls([call.run], min_reps=reps) * 1e3
        # per token: X, X' (hc*d bf16 each), delta, z (d bf16 each), post_in, comb_in, pre/post/comb out;
        # per call: hc_fn (fp32), base, scale, gamma
        nbytes = N_TOK * (2 * hc * D * 2 + 2 * D * 2 + (hc + hc * hc) * 4 + (2 * hc + hc * hc) * 4) \
            + mix * hc * D * 4 + mix * 4 + 12 + D * 4
        out[f"hc{hc}"] = {"call_us": round(us, 2), "algorithmic_bytes": nbytes,
                          "gbs": round(nbytes / us / 1e3, 1), "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
        del call
        torch.cuda.empty_cache()
    return {"workload": "fused sublayer boundary at other stream counts, B=1 T=4096, d=5120, sinkhorn_iters=20, "
                        "RMSNorm, read with the freshly derived pre", **out}


def sweep(dev, ns=(128, 512, 4096, 32768), reps=50):
    """The boundary (write, RMSNorm; hc=4, d=5120) at several token counts,
    in both read modes: one GPU's share of a batch sharded over tokens.
    n=32768 is the channel-outlier stress workload, the others prefixes of
    the prefill workload.  Event-timed over at least reps calls (after a
    warm-up) on two rotating buffer sets."""
    out = {}
    for n in ns:
        print(f"[bench] timing n={n}", file=sys.stderr, flush=True)
        s = synth.boundary_inputs("stress") if n > N_TOK else synth.boundary_inputs("prefill", 0, n)
        params = dict(fn_packed=T.hc_fn_pack(f32(s["hc_fn"], dev)), hc_base=f32(s["hc_base"], dev),
                      hc_scale=f32(s["hc_scale"], dev), gamma=f32(s["gamma"], dev))
        sets = [{k: (bf(s[k], dev) if k in ("x", "delta") else f32(s[k], dev))
                 for k in ("x", "delta", "post_in", "comb_in", "pre_in")} for _ in range(2)]
        del s
        out[str(n)] = {}
        for mode in ("lag", "fresh"):
            calls = [T.BoundaryCall(ins["x"], delta=ins["delta"], post_in=ins["post_in"], comb_in=ins["comb_in"],
                                    pre_in=ins["pre_in"] if mode == "lag" else None, **params) for ins in sets]
            us = timed_calls([c.run for c in calls], min_reps=reps) * 1e3
            nbytes = algorithmic_bytes(n, mode)
            out[str(n)][mode] = {"call_us": round(us, 2), "tokens_per_s": round(n / us * 1e6, 1),
                                 "gbs": round(nbytes / us / 1e3, 1),
                                 "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
            del calls
        del sets
        torch.cuda.empty_cache()
    return {"workload": "fused sublayer boundary, hc=4, d=5120, RMSNorm, at n tokens, given pre (lag) and fresh "
                        "pre (n=32768: channel-outlier stress inputs)", **out}


def schedules(dev, s, reps=50):
    """The given-pre call (write, read with the previous boundary's pre,
    RMSNorm; n = 4096, hc = 4, d = 5120) on its two schedules: one launch (the
    default: the workgroups of a token tile exchange their per-slice sums on
    chip, y stays in registers until its mean square is known) and two
    launches (HC_BOUNDARY_TWO_LAUNCH: per-slice records, y written and read
    back by the finishing kernel).  Event-timed like the sweep."""
    out = {}
    ins = {k: (bf(s[k], dev) if k in ("x", "delta") else f32(s[k], dev))
           for k in ("x", "delta", "post_in", "comb_in", "pre_in")}
    params = dict(fn_packed=T.hc_fn_pack(f32(s["hc_fn"], dev)), hc_base=f32(s["hc_base"], dev),
                  hc_scale=f32(s["hc_scale"], dev), gamma=f32(s["gamma"], dev))
    nbytes = algorithmic_bytes(N_TOK, "lag")
    for name, kw in (("one_launch", {}), ("two_launch", {"two_launch": True})):
        print(f"[bench] timing the given-pre call, {name}", file=sys.stderr, flush=True)
        call = T.BoundaryCall(ins["x"], delta=ins["delta"], post_in=ins["post_in"], comb_in=ins["comb_in"],
                              pre_in=ins["pre_in"], **params, **kw)
        us = timed_calls([call.run], min_reps=reps) * 1e3
        out[name] = {"call_us": round(us, 2), "gbs": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
        del call
    torch.cuda.empty_cache()
    return {"workload": "fused sublayer boundary, prefill B=1 T=4096, hc=4, d=5120, given pre, RMSNorm, "
                        "by schedule", **out}


def entry_points(dev, s, reps=50):
    """The standalone entry points on the prefill workload (n = 4096, hc = 4,
    d = 5120), each by events: hc_post, hc_pre, hc_mixes (projection + split),
    hc_split_sinkhorn.  Algorithmic bytes of each as it runs alone."""
    n = N_TOK
    X, Dl = bf(s["x"], dev), bf(s["delta"], dev)
    post, comb, pre = f32(s["post_in"], dev), f32(s["comb_in"], dev), f32(s["pre_in"], dev)
    fn = T.hc_fn_pack(f32(s["hc_fn"], dev))
    base, scale = f32(s["hc_base"], dev), f32(s["hc_scale"], dev)
    xo, y = torch.empty_like(X), torch.empty(n, D, dtype=torch.bfloat16, device=dev)
    mixes = T.hc_mixes(X, fn)
    calls = {
        "hc_post": (lambda: T.hc_post(Dl, X, post, comb, out=xo), n * (4 * D * 2 * 2 + D * 2 + 80)),
        "hc_pre": (lambda: T.hc_pre(X, pre), n * (4 * D * 2 + D * 2 + 16)),
        "hc_mixes": (lambda: T.hc_mixes(X, fn, scale, base), n * (4 * D * 2 + 96) + BYTES_CALL - D * 4),
        "hc_split_sinkhorn": (lambda: T.hc_split_sinkhorn(mixes, scale, base), n * (MIX * 4 + 96)),
    }
    out = {}
    per_graph = 20
    for name, (fn_call, nbytes) in calls.items():
        print(f"[bench] timing {name}", file=sys.stderr, flush=True)
        # the Python binding costs more per call than the small kernels take, so
        # the calls are captured in a graph (20 per replay) and the replays timed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn_call()                                    # workspace and allocator warm on this stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(per_graph):
                fn_call()
        us = timed_calls([g.replay], min_reps=max(1, reps // per_graph)) * 1e3 / per_graph
        out[name] = {"call_us": round(us, 2), "algorithmic_bytes": nbytes, "gbs": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
        del g
    del y
    return {"workload": "standalone entry points, prefill B=1 T=4096, hc=4, d=5120; 20 calls per captured "
                        "graph, replays timed by events", **out}


def stack_ends(dev, reps=50):
    """The calls at the two ends of the stand-in stack (n = 8192, hc = 4,
    d = 5120): the entry (x the embedding [n, d], read by all four streams;
    first pre 0.25 given; mixes derived; the MTP tap of the block input), a
    boundary with the tap, and the exit (last write, read with the last pre,
    RMSNorm with eps 1e-20; no mixes).  Mean microseconds per call by events."""
    st = synth.stack_inputs(2)
    n = st["h"].shape[0]
    (fn, base, scale), (fn2, base2, scale2) = st["params"]
    h = bf(st["h"], dev)
    g = f32(st["gammas"][0], dev)
    pre0 = torch.full((n, HC), 0.25, dtype=torch.float32, device=dev)
    entry = T.BoundaryCall(h, x_expanded=True, pre_in=pre0, fn_packed=T.hc_fn_pack(f32(fn, dev)),
                           hc_base=f32(base, dev), hc_scale=f32(scale, dev), gamma=g, want_mean=True)
    e = entry.outputs
    x = h.view(n, 1, D).expand(n, HC, D).contiguous()
    delta = e["y"].clone()                                   # a stand-in sublayer output
    bnd = T.BoundaryCall(x, delta=delta, post_in=e["post"], comb_in=e["comb"], pre_in=e["pre"],
                         fn_packed=T.hc_fn_pack(f32(fn2, dev)), hc_base=f32(base2, dev),
                         hc_scale=f32(scale2, dev), gamma=g, want_mean=True)
    ex = T.BoundaryCall(x, delta=delta, post_in=e["post"], comb_in=e["comb"], pre_in=e["pre"],
                        gamma=f32(st["gamma_final"], dev), rms_eps=1e-20)
    out = {}
    for name, c in (("entry_us", entry), ("boundary_with_tap_us", bnd), ("exit_us", ex)):
        print(f"[bench] timing the stack's {name[:-3]}", file=sys.stderr, flush=True)
        out[name] = round(timed_calls([c.run], min_reps=reps) * 1e3, 2)
    return {"workload": "stand-in stack ends, B=2 T=4096 (n=8192), hc=4, d=5120: expanded entry with the "
                        "MTP tap; a given-pre boundary with RMSNorm and the tap; the exit (no mixes, "
                        "RMSNorm eps 1e-20)", "tokens": n, **out}


def timed_calls(fns, min_s=0.25, min_reps=50):
    """Mean milliseconds per call of the callables fns (run in rotation),
    event-timed on the current stream.  Warms up for at least min_s (clocks
    settle), then times at least min_reps calls and at least min_s."""
    k, t0 = 0, time.perf_counter()
    while k < 20 or time.perf_counter() - t0 < min_s:
        for _ in range(10):
            fns[k % len(fns)]()
            k += 1
        torch.cuda.synchronize()
    est = (time.perf_counter() - t0) / k
    reps = max(min_reps, int(min_s / max(est, 1e-6)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fns[i % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def stats(ms):
    return {"mean": float(np.mean(ms)), "median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
            "p90": float(np.percentile(ms, 90))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--mode", choices=["lag", "fresh"], default="lag")
    ap.add_argument("--modes", default="lag,fresh", help="read modes to time (the headline mode is always timed)")
    ap.add_argument("--sets", type=int, default=4, help="rotating input/output buffer sets")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--no-copy", action="store_true", help="skip the 1 GiB reference stream")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode block timing")
    ap.add_argument("--no-other-hc", action="store_true", help="skip the hc = 2 and 8 boundary timing")
    ap.add_argument("--no-sweep", action="store_true", help="skip the token-count sweep")
    ap.add_argument("--no-stack-ends", action="store_true", help="skip the stack entry / exit timing")
    ap.add_argument("--no-entry-points", action="store_true", help="skip the standalone entry-point timing")
    ap.add_argument("--no-schedules", action="store_true", help="skip the given-pre schedules' timing")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark runs on one GPU only.  The glue is per token and would shard over "
              "tokens with no exchange between GPUs; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    print(f"[bench] generating the {N_TOK}-token prefill workload", file=sys.stderr, flush=True)
    s = synth.boundary_inputs("prefill")
    sets = make_sets(s, dev, args.sets)
    params = dict(fn_packed=T.hc_fn_pack(f32(s["hc_fn"], dev)), hc_base=f32(s["hc_base"], dev),
                  hc_scale=f32(s["hc_scale"], dev), gamma=f32(s["gamma"], dev), iters=20, hc_eps=1e-6,
                  norm_eps=1e-6, rms_eps=1e-6)
    torch.cuda.synchronize()
    settle_clocks(dev)

    results = {}
    modes = [args.mode] + [m for m in args.modes.split(",") if m and m != args.mode]
    for mode in modes:
        print(f"[bench] timing mode={mode}", file=sys.stderr, flush=True)
        r = time_mode(mode, sets, params, args.steps, args.warmup)
        nbytes = algorithmic_bytes(N_TOK, mode)
        results[mode] = {
            "wall_s": r["wall_s"], "ms_per_step": r["wall_s"] / args.steps * 1e3,
            "tokens_per_s": N_TOK * args.steps / r["wall_s"], "algorithmic_bytes": nbytes,
            "mean_call_ms": r["mean_call_ms"], "kernels": list(KERNELS[mode]),
            "gbs_at_mean_call": nbytes / (r["mean_call_ms"] * 1e-3) / 1e9,
            "frac_at_mean_call": nbytes / (r["mean_call_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "host_enqueue_us_per_call": r["host_enqueue_us_per_call"],
        }
        if "call_ms" in r:
            results[mode].update({"split_call_ms": stats(r["call_ms"]),
                                  "stream_kernel_ms": stats(r["stream_kernel_ms"]),
                                  "finish_kernel_ms": stats(r["finish_kernel_ms"])})
    ref_gbs = None if args.no_copy else reference_stream(dev)
    head = results[args.mode]
    mean_ms = head["mean_call_ms"]
    achieved = head["algorithmic_bytes"] / (mean_ms * 1e-3) / 1e9
    traffic_bytes, traffic_src = traffic(args.mode)
    dec = None if args.no_decode else {**decode_block(dev), "stack": decode_stack(dev)}
    ohc = None if args.no_other_hc else other_hc(dev)
    swp = None if args.no_sweep else sweep(dev)
    ends = None if args.no_stack_ends else stack_ends(dev)
    eps = None if args.no_entry_points else entry_points(dev, s)
    sch = None if args.no_schedules else schedules(dev, s)
    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(s, args.cpu_repeats, args.mode)

    def rnd(v):
        if isinstance(v, float):
            return round(v, 5)
        if isinstance(v, dict):
            return {k: rnd(x) for k, x in v.items()}
        return v

    line = {
        "metric": "tokens/s of fused HC sublayer boundary (T=4096); HBM GB/s as % of peak",
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 streams, fp32 arithmetic (bf16x3 split-weight MFMA projection)",
        "data": "synthetic (seeded; shapes and distributions of the prefill boundary workload)",
        "config": {"workload": "fused sublayer boundary, prefill B=1 T=4096, hc=4, d=5120, sinkhorn_iters=20, "
                               f"RMSNorm; read with the {'freshly derived' if args.mode == 'fresh' else 'previous'} pre",
                   "tokens": N_TOK, "read_mode": args.mode, "buffer_sets": args.sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_bytes,
                     "kernel": "hc_boundary = " + " + ".join(KERNELS[args.mode]),
                     "algorithmic_bytes_per_launch": head["algorithmic_bytes"],
                     "avg_launch_ms": round(mean_ms, 5),
                     **({"stream_kernel_avg_ms": round(head["stream_kernel_ms"]["mean"], 5),
                         "finish_kernel_avg_ms": round(head["finish_kernel_ms"]["mean"], 5)}
                        if "stream_kernel_ms" in head else {}),
                     "traffic_source": traffic_src},
        "cpu_baseline": cpu,
        "modes": {k: rnd(v) for k, v in results.items()},
        "reference_stream_gbs": None if ref_gbs is None else round(ref_gbs, 1),
        "decode": dec,
        "other_hc": ohc,
        "sweep": swp,
        "stack_ends": ends,
        "entry_points": eps,
        "schedules": sch,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
