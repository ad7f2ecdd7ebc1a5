"""Benchmark of FusedKV reconstruction-layer attention on one MI355X.

One step is one decode pass over every reconstruction layer of the 650M-shape
model (16 layers; layers 9..16 rebuild K/V from layers 1 and 8): 8 calls of
fkv_decode, batch 32, 8192 cached tokens, 16 query / 8 KV heads, head dim 96,
bf16, head-major caches, each layer with its own queries and fusion vectors.
`value` is the step's algorithmic cache traffic divided by its MEDIAN time
(GB/s) over --steps repetitions (default 50) after --warmup untimed ones
(default 10); every repetition is bracketed by HIP events on the stream the
library calls are enqueued on, and p10 / p90 / mean are reported beside the
median.  The roofline block divides the algorithmic bytes of one launch of
the four-source decode kernel by its mean single-launch duration (an event
pair around each launch).

Beside it the line reports
  * the Lite and plain-control decode variants, each also replayed as one
    HIP graph, and the fp64 oracle timed on the host cores on a bounded
    sample of the decode workload (cpu_baseline);
  * the causal prefill of the 1.5B shape (batch 4, S = 8192, 16/8 heads,
    D = 128, 12 fused layers), tiles fused inside the attention kernel, in
    TFLOP/s with its own roofline block and the oracle on sampled query rows
    of one layer (prefill.cpu_baseline);
  * next_rows: the whole-stack decode at batch 1 and 131072 cached tokens
    (FusedKV, Lite and an all-plain model as HIP graphs: time and byte ratios
    over the plain model), attention time to first token over an 8192-token
    prompt (FusedKV schedule over the plain model), and the HBM fractions of
    the G = 64 decode and of the decode over 4-bit sources;
  * device: name, CU count, and the engine / memory clocks that rocm-smi
    reported while the bench ran.

Algorithmic work (what the method must move or compute, per layer call):
  decode  bytes = 4*B*S*Hkv*D*2 (four bf16 source caches; 2 for Lite/vanilla)
                  + 2*B*Hq*D*2 (Q, O) + 16*Hkv*D (fp32 weights)
  prefill flops = 2*D*S*(S+1)*B*Hq (QK^T and PV over the causal triangle)
Inputs are synthetic and seeded (see cross_layer_kv_amd/inputs.py) and
resident in HBM before timing starts.

`--workload NAME` measures one of the other configured workloads instead and
prints one JSON line for it: tiny-decode (fp32, cache-resident correctness
shape), 4b-decode, hgqa-decode (64 query heads per KV head, matrix-core
kernel), kivi-decode (4-bit sources), 4b-prefill, 1.5b-prefill,
1.5b-prefill-bwd (backward), long-decode-b1 / long-decode-b8 (131072 cached
tokens; the whole 24-layer stack: 12 storage layers of plain attention plus
12 reconstruction layers, FusedKV vs Lite vs an all-plain model, each step
replayed as one HIP graph, with the eager time beside it), and 1.5b-ttft
(time to first token over the attention of all 24 layers: each storage layer
writes its new keys and values into its caches and runs causal prefill over
them; the reconstruction layers run only the final query row, a decode at S
over the caches of layers 1 and 12; against 24 storage layers).
`--part decode|prefill|next` runs one part of the default line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)

DECODE = dict(name="650M-shape FusedKV decode, layers 9-16 fused from layers 1 and 8",
              B=32, S=8192, Hq=16, Hkv=8, D=96, layers=8, seed=0xF0002)
PREFILL = dict(name="1.5B-shape FusedKV causal prefill, layers 13-24 fused from layers 1 and 12",
               B=4, S=8192, Hq=16, Hkv=8, D=128, layers=12, seed=0xF0003)


WORKLOADS = {
    "tiny-decode": dict(kind="decode", name="tiny FusedKV decode (fp32, one layer, cache-resident)",
                        B=1, S=1024, Hq=4, Hkv=2, D=64, layers=1, seed=0xF0001, dtype="f32"),
    "650m-decode": dict(kind="decode", **DECODE),
    "4b-decode": dict(kind="decode", name="4B-shape FusedKV decode, layers 19-36 fused from layers 1 and 18",
                      B=16, S=32768, Hq=32, Hkv=16, D=80, layers=18, seed=0xF0004),
    "hgqa-decode": dict(kind="decode", name="high-GQA FusedKV decode (128 query heads over 2 KV heads, G=64), 8 layers",
                        B=16, S=32768, Hq=128, Hkv=2, D=128, layers=8, seed=0xF0006),
    "1.5b-prefill": dict(kind="prefill", **PREFILL),
    "1.5b-prefill-bwd": dict(kind="backward", name="1.5B-shape FusedKV causal prefill backward (dQ, source and "
                             "fusion-weight gradients), layers 13-24", B=4, S=8192, Hq=16, Hkv=8, D=128, layers=12,
                             seed=0xF0003),
    "4b-prefill": dict(kind="prefill", name="4B-shape FusedKV causal prefill, layers 19-36 fused from layers 1 and 18",
                       B=1, S=16384, Hq=32, Hkv=16, D=80, layers=18, seed=0xF0004),
    "long-decode-b1": dict(kind="stack", name="1.5B-shape long-context decode, whole 24-layer stack, batch 1",
                           B=1, S=131072, Hq=16, Hkv=8, D=128, layers=12, seed=0xF0005),
    "long-decode-b8": dict(kind="stack", name="1.5B-shape long-context decode, whole 24-layer stack, batch 8",
                           B=8, S=131072, Hq=16, Hkv=8, D=128, layers=12, seed=0xF0005),
    "kivi-decode": dict(kind="kivi", name="650M-shape FusedKV decode over 4-bit (KIVI-style) source caches, 8 layers",
                        B=32, S=8192, Hq=16, Hkv=8, D=96, layers=8, seed=0xF0007),
    "1.5b-ttft": dict(kind="ttft", name="1.5B-shape attention time to first token, 24 layers, 8192-token prompt",
                      B=1, S=8192, Hq=16, Hkv=8, D=128, layers=12, seed=0xF0003),
}


def source_sha(*names):
    """sha256[:16] over kernel sources under cross_layer_kv_amd/csrc."""
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "cross_layer_kv_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


# committed counter summaries: file, the sources whose hash they were taken
# on, and the key holding the HBM bytes per launch of the timed kernel
TRAFFIC = {
    "decode": ("decode_650m_bf16_hbm_traffic.txt", ("fkv_decode.hip", "fkv_internal.h"), "traffic_bytes_per_launch"),
    "kivi": ("kivi_decode_650m_4bit_hbm_traffic.txt", ("fkv_kivi.hip", "fkv_mfma_common.h", "fkv_internal.h"),
             "traffic_bytes_per_launch"),
    "prefill": ("prefill_1p5b_bf16_hbm_traffic.txt", ("fkv_prefill.hip", "fkv_mfma_common.h", "fkv_internal.h"),
                "traffic_bytes_per_launch"),
}


def recorded_traffic(which):
    """HBM bytes per launch of a kernel from its committed counter summary
    (FETCH_SIZE and WRITE_SIZE runs scaled by a copy kernel of known size);
    None when the kernel's sources changed since the counters were taken, or
    when there is no summary."""
    fname, srcs, key = TRAFFIC[which]
    try:
        text = open(os.path.join(ROOT, "profiles", fname), encoding="utf-8").read()
        sha = source_sha(*srcs)
    except OSError:
        return None
    fields = {}
    for ln in text.splitlines():
        if ln and not ln.startswith("#") and ":" in ln:
            k, v = ln.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != sha or key not in fields:
        return None
    return int(fields[key])


def decode_bytes(B, S, Hq, Hkv, D, sources, elt=2):
    return sources * B * S * Hkv * D * elt + 2 * B * Hq * D * elt + (16 * Hkv * D if sources == 4 else 0)


def kivi_decode_bytes(B, S, Hq, Hkv, D, sources):
    """Algorithmic bytes of one 4-bit decode launch: per source the codes
    (D/2 bytes a token) and fp16 scale + minimum (keys per 32-token group
    and channel, values per token and 32-channel group), plus Q and O
    (bf16) and, fused, the four float32 weight vectors."""
    codes = B * Hkv * S * D // 2
    kmeta = B * Hkv * ((S + 31) // 32) * D * 4
    vmeta = B * Hkv * S * ((D + 31) // 32) * 4
    per_pair = 2 * codes + kmeta + vmeta
    return per_pair * (sources // 2) + 2 * B * Hq * D * 2 + (16 * Hkv * D if sources == 4 else 0)


def prefill_flops(B, S, Hq, D):
    return 2 * D * S * (S + 1) * B * Hq


def _pct(sorted_vals, p):
    """p-th percentile (linear interpolation between order statistics)."""
    n = len(sorted_vals)
    x = (n - 1) * p / 100.0
    i = int(x)
    j = min(i + 1, n - 1)
    return sorted_vals[i] + (sorted_vals[j] - sorted_vals[i]) * (x - i)


def _stats(ms):
    a = sorted(ms)
    return dict(median_ms=_pct(a, 50), p10_ms=_pct(a, 10), p90_ms=_pct(a, 90), mean_ms=sum(a) / len(a),
                min_ms=a[0], max_ms=a[-1], reps=len(a))


# wall-clock windows (time.time()) of the timed GPU regions, used to tell
# clock samples taken while the GPU was busy from the others
BUSY = []


def _time_steps(fn, reps, warmup, stream):
    """`warmup` untimed calls of fn, then `reps` calls, each bracketed by HIP
    events recorded on `stream` (the stream every library call here is
    enqueued on), back to back: per-call durations with no host gap counted
    twice.  Synchronised on both sides."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    t0 = time.time()
    ev[0].record(stream)
    for i in range(reps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    BUSY.append((t0, time.time()))
    return _stats([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])


def _time_launches(launches, reps, warmup, stream):
    """Durations of single launches: each callable in `launches` enqueues one
    kernel launch (one library call), and an event pair on `stream` brackets
    every one of them over `reps` passes of the list."""
    import torch
    for _ in range(warmup):
        for f in launches:
            f()
    torch.cuda.synchronize()
    n = len(launches)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n * reps)]
    k = 0
    t0 = time.time()
    for _ in range(reps):
        for f in launches:
            ev[k].record(stream)
            f()
            ev[k + 1].record(stream)
            k += 2
    torch.cuda.synchronize()
    BUSY.append((t0, time.time()))
    return _stats([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n * reps)])


def _capture(fn, stream):
    """fn(st) (a sequence of library calls on stream st) captured as one HIP
    graph.  It runs once on the capture stream first, so nothing is set up
    during capture; the library records only kernel launches."""
    import torch
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        fn(cap)
    cap.synchronize()
    with torch.cuda.graph(g, stream=cap):
        fn(cap)
    torch.cuda.synchronize()
    return g


def _variant(st, byts, nl, launch=None, graph=None, flops=False):
    """Per-variant record: the step statistics, the throughput at the median
    step, per-layer time, and (when timed) single-launch and graph-replay
    statistics."""
    med = st["median_ms"] * 1e-3
    r = dict(step=st, ms_per_step=st["median_ms"], ms_per_layer=st["median_ms"] / nl, work_per_step=byts)
    r["rate"] = byts / med / (1e12 if flops else 1e9)
    if launch is not None:
        r["launch"] = launch
        r["launch_rate"] = byts / nl / (launch["mean_ms"] * 1e-3) / (1e12 if flops else 1e9)
    if graph is not None:
        r["graph"] = graph
        r["graph_rate"] = byts / (graph["median_ms"] * 1e-3) / (1e12 if flops else 1e9)
    return r


def run_decode(cfg, steps, warmup, stream, variants=("fused", "lite", "vanilla"), graphs=True):
    import torch
    from cross_layer_kv_amd import binding, inputs
    dev = "cuda:0"
    B, S, Hq, Hkv, D, nl = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["layers"]
    dt = torch.float32 if cfg.get("dtype") == "f32" else torch.bfloat16
    base = inputs.make_layer(B, 1, S, Hq, Hkv, D, dt, cfg["seed"], dev)
    qs = [inputs.make_queries(B, 1, Hq, D, dt, cfg["seed"] * 97 + i, dev,
                              positions=torch.full((1,), S - 1)) for i in range(nl)]
    ws_list = [inputs.make_weights(Hkv, D, cfg["seed"] * 89 + i, device=dev) for i in range(nl)]
    outs = [torch.empty_like(q) for q in qs]
    ws = binding.decode_workspace(qs[0], base.k1)

    def fused(i, st=stream):
        binding.fkv_decode(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], out=outs[i], workspace=ws,
                           stream=st)

    def lite(i, st=stream):
        binding.fkv_lite_decode(qs[i], base.kn, base.v1, out=outs[i], workspace=ws, stream=st)

    def vanilla(i, st=stream):  # storage-layer control: attention over a layer's own caches
        k, v = (base.k1, base.v1) if i % 2 == 0 else (base.kn, base.vn)
        binding.fkv_lite_decode(qs[i], k, v, out=outs[i], workspace=ws, stream=st)

    layer_fns = {"fused": fused, "lite": lite, "vanilla": vanilla}
    srcs = {"fused": 4, "lite": 2, "vanilla": 2}
    res = {}
    elt = 4 if dt == torch.float32 else 2
    for name in variants:
        lf = layer_fns[name]

        def step(st=stream, lf=lf):
            for i in range(nl):
                lf(i, st)

        byts = decode_bytes(B, S, Hq, Hkv, D, srcs[name], elt) * nl
        st = _time_steps(step, steps, warmup, stream)
        launch = _time_launches([lambda i=i, lf=lf: lf(i) for i in range(nl)], max(5, steps // 5), 2, stream) \
            if name == "fused" else None
        graph = None
        if graphs:
            # the same step replayed as one HIP graph: no host launch cost between kernels
            g = _capture(step, stream)
            graph = _time_steps(g.replay, steps, warmup, stream)
            del g
        res[name] = _variant(st, byts, nl, launch, graph)
        res[name]["bytes_per_layer"] = byts // nl
    return res, base


def run_kivi(cfg, steps, warmup, stream, variants=("fused", "lite", "bf16_fused")):
    """4-bit decode: the caches are quantised once (outside the timed
    region, as a prefill would write them); one step is `layers` fused
    decode launches.  The bf16 fused decode on the same sources is timed
    beside it."""
    import torch
    from cross_layer_kv_amd import binding, inputs
    dev = "cuda:0"
    B, S, Hq, Hkv, D, nl = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["layers"]
    base = inputs.make_layer(B, 1, S, Hq, Hkv, D, torch.bfloat16, cfg["seed"], dev)
    names = ("k1", "kn", "v1", "vn")
    q4 = {n: binding.fkv_kivi_quantize(getattr(base, n), n in ("v1", "vn")) for n in names}
    qs = [inputs.make_queries(B, 1, Hq, D, torch.bfloat16, cfg["seed"] * 97 + i, dev,
                              positions=torch.full((1,), S - 1)) for i in range(nl)]
    ws_list = [inputs.make_weights(Hkv, D, cfg["seed"] * 89 + i, device=dev) for i in range(nl)]
    outs = [torch.empty_like(q) for q in qs]
    ws = binding.decode_workspace(qs[0], base.k1)

    def quantise_step():
        for n in names:
            binding.fkv_kivi_quantize(getattr(base, n), n in ("v1", "vn"), dst=q4[n], stream=stream)

    def fused(i):
        binding.fkv_kivi_decode(qs[i], q4["k1"], q4["kn"], q4["v1"], q4["vn"], ws_list[i], out=outs[i],
                                workspace=ws, stream=stream)

    def lite(i):
        binding.fkv_kivi_lite_decode(qs[i], q4["kn"], q4["v1"], out=outs[i], workspace=ws, stream=stream)

    def bf16_fused(i):
        binding.fkv_decode(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], out=outs[i], workspace=ws,
                           stream=stream)

    fns = {"fused": (fused, kivi_decode_bytes(B, S, Hq, Hkv, D, 4)),
           "lite": (lite, kivi_decode_bytes(B, S, Hq, Hkv, D, 2)),
           "bf16_fused": (bf16_fused, decode_bytes(B, S, Hq, Hkv, D, 4))}
    res = {}
    for name in variants:
        lf, per = fns[name]

        def step(lf=lf):
            for i in range(nl):
                lf(i)

        st = _time_steps(step, steps, warmup, stream)
        launch = _time_launches([lambda i=i, lf=lf: lf(i) for i in range(nl)], max(5, steps // 5), 2, stream) \
            if name == "fused" else None
        res[name] = _variant(st, per * nl, nl, launch)
        res[name]["bytes_per_layer"] = per
    if "fused" in variants and "lite" in variants:
        qs_ = _time_steps(quantise_step, 5, 1, stream)
        res["quantise"] = dict(ms_per_source=qs_["median_ms"] / 4,
                               gbs=B * S * Hkv * D * 2 / (qs_["median_ms"] / 4 * 1e-3) / 1e9)
    return res


def run_prefill(cfg, steps, warmup, stream, keep_base=False):
    import torch
    from cross_layer_kv_amd import binding, inputs
    dev = "cuda:0"
    B, S, Hq, Hkv, D, nl = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["layers"]
    base = inputs.make_layer(B, S, S, Hq, Hkv, D, torch.bfloat16, cfg["seed"], dev, decode=False)
    qs = [base.q] + [inputs.make_queries(B, S, Hq, D, torch.bfloat16, cfg["seed"] * 97 + i, dev)
                     for i in range(1, nl)]
    ws_list = [base.weights] + [inputs.make_weights(Hkv, D, cfg["seed"] * 89 + i, device=dev)
                                for i in range(1, nl)]
    out = torch.empty_like(base.q)

    # every attention workgroup fuses (or, single-source, converts) the
    # tiles it reads inside the kernel; nothing is staged in memory
    def fused(i):
        binding.fkv_prefill(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], out=out, causal=True,
                            stream=stream)

    def lite(i):
        binding.fkv_lite_prefill(qs[i], base.kn, base.v1, out=out, causal=True, stream=stream)

    res = {}
    fl = prefill_flops(B, S, Hq, D)
    for name, lf in (("fused", fused), ("lite", lite)):
        def step(lf=lf):
            for i in range(nl):
                lf(i)

        st = _time_steps(step, steps, warmup, stream)
        launch = _time_launches([lambda i=i, lf=lf: lf(i) for i in range(nl)], max(3, steps // 10), 1, stream)
        res[name] = _variant(st, fl * nl, nl, launch, flops=True)
    del qs, out
    torch.cuda.empty_cache()
    return res, (base if keep_base else None)


def backward_flops(B, S, Hq, D):
    """Five products (recomputed scores, dP, dV, dQ, dK) over the causal
    triangle including the diagonal, FMA = 2: 2.5 x the forward's."""
    return 5 * D * S * (S + 1) * B * Hq


def run_backward(cfg, steps, warmup, stream):
    """One step = `layers` backward calls (distinct queries, output
    gradients and weights per layer) over the same four sources; the forward
    outputs and LSEs they consume are computed once, untimed."""
    import torch
    from cross_layer_kv_amd import binding, inputs
    dev = "cuda:0"
    B, S, Hq, Hkv, D, nl = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["layers"]
    base = inputs.make_layer(B, S, S, Hq, Hkv, D, torch.bfloat16, cfg["seed"], dev, decode=False)
    qs = [base.q] + [inputs.make_queries(B, S, Hq, D, torch.bfloat16, cfg["seed"] * 97 + i, dev)
                     for i in range(1, nl)]
    ws_list = [base.weights] + [inputs.make_weights(Hkv, D, cfg["seed"] * 89 + i, device=dev)
                                for i in range(1, nl)]
    douts = [inputs.make_grad_output(B, S, Hq, D, torch.bfloat16, cfg["seed"] * 83 + i, dev) for i in range(nl)]
    fwd = {"fused": [], "lite": []}
    for i in range(nl):
        o, l = torch.empty_like(qs[i]), torch.empty(B, Hq, S, dtype=torch.float32, device=dev)
        binding.fkv_prefill(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], out=o, lse=l, causal=True)
        fwd["fused"].append((o, l))
        o, l = torch.empty_like(qs[i]), torch.empty(B, Hq, S, dtype=torch.float32, device=dev)
        binding.fkv_lite_prefill(qs[i], base.kn, base.v1, out=o, lse=l, causal=True)
        fwd["lite"].append((o, l))
    dq = torch.empty_like(base.q)
    grads = [torch.empty(B, S, Hkv, D, dtype=torch.bfloat16, device=dev) for _ in range(4)]
    dw = [torch.empty(Hkv, D, dtype=torch.float32, device=dev) for _ in range(4)]
    ws = binding.backward_workspace(base.q, base.k1)

    def fused(i):
        o, l = fwd["fused"][i]
        binding.fkv_prefill_backward(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], o, l, douts[i],
                                     dq=dq, dk1=grads[0], dkn=grads[1], dv1=grads[2], dvn=grads[3], dweights=dw,
                                     workspace=ws, causal=True, stream=stream)

    def lite(i):
        o, l = fwd["lite"][i]
        binding.fkv_lite_prefill_backward(qs[i], base.kn, base.v1, o, l, douts[i], dq=dq, dk=grads[0],
                                          dv=grads[2], workspace=ws, causal=True, stream=stream)

    res = {}
    fl = backward_flops(B, S, Hq, D)
    for name, lf in (("fused", fused), ("lite", lite)):
        def step(lf=lf):
            for i in range(nl):
                lf(i)

        st = _time_steps(step, steps, warmup, stream)
        res[name] = _variant(st, fl * nl, nl, flops=True)
    del qs, douts, fwd, base
    torch.cuda.empty_cache()
    return res


def run_stack(cfg, steps, warmup, stream):
    """One decode step through the whole 2n-layer stack: n storage layers of
    plain attention over their own caches, then n reconstruction layers
    (FusedKV or Lite), against an all-vanilla model of 2n plain layers.
    Storage layers rotate over four distinct cache pairs (each far larger
    than the 256 MB last-level cache), so every layer streams from HBM."""
    import torch
    from cross_layer_kv_amd import binding, inputs
    dev = "cuda:0"
    B, S, Hq, Hkv, D, nl = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["layers"]
    base = inputs.make_layer(B, 1, S, Hq, Hkv, D, torch.bfloat16, cfg["seed"], dev)
    extra = [(inputs.make_cache(B, S, Hkv, D, torch.bfloat16, cfg["seed"] * 31 + 2 * i, dev),
              inputs.make_cache(B, S, Hkv, D, torch.bfloat16, cfg["seed"] * 31 + 2 * i + 1, dev, rotate=False))
             for i in range(2)]
    pairs = [(base.k1, base.v1), (base.kn, base.vn)] + extra
    qs = [inputs.make_queries(B, 1, Hq, D, torch.bfloat16, cfg["seed"] * 97 + i, dev,
                              positions=torch.full((1,), S - 1)) for i in range(2 * nl)]
    ws_list = [inputs.make_weights(Hkv, D, cfg["seed"] * 89 + i, device=dev) for i in range(nl)]
    out = torch.empty_like(qs[0])
    ws = binding.decode_workspace(qs[0], base.k1)

    def storage(i, st):
        k, v = pairs[i % 4]
        binding.fkv_lite_decode(qs[i], k, v, out=out, workspace=ws, stream=st)

    def fused_model(st=stream):
        for i in range(nl):
            storage(i, st)
        for i in range(nl):
            binding.fkv_decode(qs[nl + i], base.k1, base.kn, base.v1, base.vn, ws_list[i], out=out,
                               workspace=ws, stream=st)

    def lite_model(st=stream):
        for i in range(nl):
            storage(i, st)
        for i in range(nl):
            binding.fkv_lite_decode(qs[nl + i], base.kn, base.v1, out=out, workspace=ws, stream=st)

    def vanilla_model(st=stream):
        for i in range(2 * nl):
            storage(i, st)

    per_layer = decode_bytes(B, S, Hq, Hkv, D, 2)
    res = {}
    for name, fn, byts in (("fused", fused_model, nl * per_layer + nl * decode_bytes(B, S, Hq, Hkv, D, 4)),
                           ("lite", lite_model, 2 * nl * per_layer),
                           ("vanilla", vanilla_model, 2 * nl * per_layer)):
        eager = _time_steps(fn, steps, warmup, stream)
        # the whole step as one HIP graph, replayed on the timing stream
        g = _capture(fn, stream)
        gst = _time_steps(g.replay, steps, warmup, stream)
        del g
        res[name] = dict(step=gst, ms_per_step=gst["median_ms"], gbs=byts / (gst["median_ms"] * 1e-3) / 1e9,
                         bytes=byts, eager=eager)
    del base, extra, pairs
    torch.cuda.empty_cache()
    return res


def run_ttft(cfg, steps, warmup, stream):
    """Attention time to first token of a 2n-layer model over an S-token
    prompt.  Every storage layer first writes its new keys and values
    (token-major, as a projection leaves them) into its head-major caches,
    then runs causal prefill over those caches.  FusedKV reconstruction
    layers need only the final prompt position: one decode at S over the
    caches that layers 1 and n have just written.  The plain model runs the
    storage-layer work (write + causal prefill) in all 2n layers."""
    import torch
    from cross_layer_kv_amd import binding, inputs
    dev = "cuda:0"
    B, S, Hq, Hkv, D, nl = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["layers"]
    qfull = inputs.make_queries(B, S, Hq, D, torch.bfloat16, cfg["seed"] * 16 + 5, dev)
    qlast = qfull[:, S - 1:S].contiguous()
    out_full = torch.empty_like(qfull)
    out_last = torch.empty_like(qlast)
    # new rows of the layers (token-major projection output); two distinct
    # sets alternate over the layers
    new = [(inputs.make_cache(B, S, Hkv, D, torch.bfloat16, cfg["seed"] * 16 + 1 + 2 * j, dev, layout="bshd"),
            inputs.make_cache(B, S, Hkv, D, torch.bfloat16, cfg["seed"] * 16 + 2 + 2 * j, dev, layout="bshd",
                              rotate=False)) for j in range(2)]
    # one head-major cache pair per layer of the plain model (the FusedKV
    # model uses the first n)
    caches = [(torch.empty(B, Hkv, S, D, dtype=torch.bfloat16, device=dev).transpose(1, 2),
               torch.empty(B, Hkv, S, D, dtype=torch.bfloat16, device=dev).transpose(1, 2)) for _ in range(2 * nl)]
    w = inputs.make_weights(Hkv, D, cfg["seed"] * 16 + 6, device=dev)
    ws = binding.decode_workspace(qlast, caches[0][0])

    def storage_layer(i):
        kn, vn = new[i % 2]
        kc, vc = caches[i]
        binding.fkv_store_kv(kn, vn, kc, vc, stream=stream)
        binding.fkv_lite_prefill(qfull, kc, vc, out=out_full, causal=True, stream=stream)

    def vanilla_model():
        for i in range(2 * nl):
            storage_layer(i)

    def fused_model():
        for i in range(nl):
            storage_layer(i)
        (k1, v1), (kn_, vn_) = caches[0], caches[nl - 1]
        for i in range(nl):
            binding.fkv_decode(qlast, k1, kn_, v1, vn_, w, out=out_last, workspace=ws, stream=stream)

    res = {}
    for name, fn in (("vanilla", vanilla_model), ("fused", fused_model)):
        st = _time_steps(fn, steps, warmup, stream)
        res[name] = dict(step=st, ms=st["median_ms"])
    del caches, new
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg, base, budget_s=12.0):
    """The fp64 oracle (unchanged) on the host cores, on whole layers of the
    decode workload: one layer at a time until ~budget_s seconds of CPU work
    have passed."""
    import oracle
    from cross_layer_kv_amd import inputs
    h = inputs.host_array
    q, k1, kn, v1, vn = (h(t) for t in (base.q, base.k1, base.kn, base.v1, base.vn))
    w = [x.cpu().numpy() for x in base.weights]
    B, S, Hq, Hkv, D = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    # bounded sample: a prefix of the batch sized so one repetition is short
    t0 = time.perf_counter()
    oracle.attend(q[:1], k1[:1], v1[:1], kn[:1], vn[:1], k_w1=w[0], k_wn=w[1], v_w1=w[2], v_wn=w[3])
    one = time.perf_counter() - t0
    nb = int(max(1, min(B, budget_s / max(one, 1e-3) / 2)))
    reps, elapsed = 0, 0.0
    t0 = time.perf_counter()
    while elapsed < budget_s or reps == 0:
        oracle.attend(q[:nb], k1[:nb], v1[:nb], kn[:nb], vn[:nb], k_w1=w[0], k_wn=w[1], v_w1=w[2], v_wn=w[3])
        reps += 1
        elapsed = time.perf_counter() - t0
    byts = decode_bytes(nb, S, Hq, Hkv, D, 4) * reps
    return dict(value=round(byts / elapsed / 1e9, 4), unit="GB/s", cores=oracle.num_threads(), kind="oracle",
                sample="%d x one fused decode layer on batch rows 0..%d of the 650M-shape workload "
                       "(S=%d, %d/%d heads, D=%d), %.1f s" % (reps, nb - 1, S, Hq, Hkv, D, elapsed))


def cpu_baseline_prefill(cfg, base, budget_s=12.0):
    """The fp64 oracle (unchanged) on sampled query rows of one causal
    prefill layer of the workload (layer 13: queries and weights of the
    first timed layer).  Rows (b, h, p) are taken with positions spread
    evenly over the prompt, batch rows and heads cycling, until ~budget_s
    seconds of CPU work; the rate counts each row's algorithmic flops,
    4 * D * (p + 1) (scores and PV over its causal prefix)."""
    import numpy as np
    import oracle
    from cross_layer_kv_amd import inputs
    h = inputs.host_array
    q, k1, kn, v1, vn = (h(t) for t in (base.q, base.k1, base.kn, base.v1, base.vn))
    w = [x.cpu().numpy() for x in base.weights]
    B, S, Hq, D = cfg["B"], cfg["S"], cfg["Hq"], cfg["D"]

    def rows_of(n, offset):
        j = np.arange(n) + offset
        # golden-ratio stride over the positions, so successive batches of
        # rows cover the prompt evenly
        p = (np.floor(((j * 0.6180339887498949) % 1.0) * S)).astype(np.int64)
        b, hh = j % B, (j // B) % Hq
        return oracle.row_index(b, hh, p, Hq, S), p

    def run(rows):
        oracle.attend(q, k1, v1, kn, vn, k_w1=w[0], k_wn=w[1], v_w1=w[2], v_wn=w[3], causal=True, rows=rows)

    r, p = rows_of(16, 0)
    t0 = time.perf_counter()
    run(r)
    one = time.perf_counter() - t0
    n = int(max(16, min(4096, 16 * (budget_s / 4) / max(one, 1e-3))))
    done, flops, elapsed, off = 0, 0, 0.0, 16
    t0 = time.perf_counter()
    while elapsed < budget_s or done == 0:
        r, p = rows_of(n, off)
        run(r)
        off += n
        done += n
        flops += int(np.sum(4 * D * (p + 1)))
        elapsed = time.perf_counter() - t0
    return dict(value=round(flops / elapsed / 1e12, 6), unit="TFLOP/s", cores=oracle.num_threads(), kind="oracle",
                sample="%d query rows (b, h, p) of one fused causal prefill layer of the 1.5B-shape workload "
                       "(B=%d, S=%d, %d/%d heads, D=%d), positions spread evenly over the prompt, %.1f s"
                       % (done, B, S, Hq, cfg["Hkv"], D, elapsed))


# A child process started before this process touches the GPU polls the
# engine and memory clocks with rocm-smi every two seconds while the bench
# runs (it never forks from a process that has initialised the GPU).
_CLOCK_SAMPLER = r"""
import json, shutil, subprocess, sys, time
exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
while True:
    t0 = time.time()
    try:
        r = subprocess.run([exe, "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        out, err = (r.stdout, "") if r.returncode == 0 else ("", (r.stderr or r.stdout)[-200:])
    except Exception as e:
        out, err = "", repr(e)[-200:]
    print(json.dumps({"t0": t0, "t": time.time(), "out": out, "err": err}), flush=True)
    time.sleep(2.0)
"""


def start_clock_sampler():
    import subprocess
    try:
        return subprocess.Popen([sys.executable, "-c", _CLOCK_SAMPLER], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None


def stop_clock_sampler(proc):
    """Stop the sampler (its own PID) and summarise the clocks it saw: per
    clock domain the min / median / max MHz over all samples, and over the
    samples whose query overlapped a timed GPU region ("busy")."""
    import re
    if proc is None:
        return {"clocks": "unavailable: sampler did not start"}
    proc.terminate()
    try:
        text, _ = proc.communicate(timeout=10)
    except Exception:
        proc.kill()
        text, _ = proc.communicate()
    seen, busy, errs, n = {}, {}, [], 0
    for ln in (text or "").splitlines():
        try:
            rec = json.loads(ln)
        except ValueError:
            continue
        n += 1
        if not rec.get("out"):
            errs.append(rec.get("err", ""))
            continue
        try:
            cards = json.loads(rec["out"])
        except ValueError:
            errs.append("unparsed rocm-smi output")
            continue
        t0, t1 = rec.get("t0", rec.get("t", 0)), rec.get("t", 0)
        in_busy = any(a < t1 and t0 < b for a, b in BUSY)
        for card, fields in cards.items():
            if not isinstance(fields, dict):
                continue
            for k, v in fields.items():
                m = re.search(r"(\d+)\s*Mhz", str(v), re.I)
                if m and "speed" in k.lower():
                    seen.setdefault(k.split()[0].lower(), []).append(int(m.group(1)))
                    if in_busy:
                        busy.setdefault(k.split()[0].lower(), []).append(int(m.group(1)))
    if not seen:
        return {"clocks": "unavailable: " + (errs[-1] if errs else "no samples"), "clock_samples": n}
    out = {}
    for dom, vals in sorted(seen.items()):
        v = sorted(vals)
        out[dom + "_mhz"] = {"min": v[0], "median": v[len(v) // 2], "max": v[-1]}
        b = sorted(busy.get(dom, []))
        if b:
            out[dom + "_mhz"]["busy"] = {"min": b[0], "median": b[len(b) // 2], "max": b[-1], "samples": len(b)}
    return {"clocks": out, "clock_samples": n, "clock_source": "rocm-smi --showclocks, sampled every 2 s during the run"}


def _stats_out(st):
    return {"median_ms": round(st["median_ms"], 4), "p10_ms": round(st["p10_ms"], 4),
            "p90_ms": round(st["p90_ms"], 4), "mean_ms": round(st["mean_ms"], 4), "reps": st["reps"]}


def _decode_block(res):
    out = {}
    for k, v in res.items():
        out[k] = {"GB/s": round(v["rate"], 2), "us_per_layer": round(v["ms_per_layer"] * 1e3, 2),
                  "frac": round(v["rate"] / HBM_PEAK_GBS, 4), "step": _stats_out(v["step"])}
        if "graph" in v:
            out[k]["graph_GB/s"] = round(v["graph_rate"], 2)
            out[k]["graph_step"] = _stats_out(v["graph"])
    return out


def _hbm_roofline(v, kernel, traffic):
    """Roofline of the timed kernel from its single-launch statistics:
    algorithmic bytes per launch / mean launch duration."""
    ach = v["bytes_per_layer"] / (v["launch"]["mean_ms"] * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "bytes_per_launch": v["bytes_per_layer"],
            "avg_launch_us": round(v["launch"]["mean_ms"] * 1e3, 2),
            "median_launch_us": round(v["launch"]["median_ms"] * 1e3, 2),
            "p10_launch_us": round(v["launch"]["p10_ms"] * 1e3, 2),
            "p90_launch_us": round(v["launch"]["p90_ms"] * 1e3, 2), "launches_timed": v["launch"]["reps"]}


def _mfma_roofline(v, kernel, flops_per_launch, traffic=None):
    ach = flops_per_launch / (v["launch"]["mean_ms"] * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "flops_per_launch": flops_per_launch, "avg_launch_us": round(v["launch"]["mean_ms"] * 1e3, 2),
            "median_launch_us": round(v["launch"]["median_ms"] * 1e3, 2),
            "p10_launch_us": round(v["launch"]["p10_ms"] * 1e3, 2),
            "p90_launch_us": round(v["launch"]["p90_ms"] * 1e3, 2), "launches_timed": v["launch"]["reps"]}


def next_rows(steps, warmup, stream):
    """Compact figures of the rows beyond the headline step, each from its
    own workload: the whole-stack decode ratio at batch 1 and 131072 cached
    tokens, attention TTFT of the FusedKV schedule over the plain model, and
    the HBM fractions of the G = 64 decode and of the 4-bit decode."""
    import torch
    out = {}
    cfg = WORKLOADS["long-decode-b1"]
    print("bench: %s" % cfg["name"], file=sys.stderr, flush=True)
    st = run_stack(cfg, steps, warmup, stream)
    out["stack_b1_s131072"] = {"fused_over_vanilla_time": round(st["fused"]["ms_per_step"] / st["vanilla"]["ms_per_step"], 3),
                               "lite_over_vanilla_time": round(st["lite"]["ms_per_step"] / st["vanilla"]["ms_per_step"], 3),
                               "fused_over_vanilla_bytes": round(st["fused"]["bytes"] / st["vanilla"]["bytes"], 3),
                               "fused_ms": round(st["fused"]["ms_per_step"], 4),
                               "vanilla_ms": round(st["vanilla"]["ms_per_step"], 4),
                               "fused_frac": round(st["fused"]["gbs"] / HBM_PEAK_GBS, 4)}
    cfg = WORKLOADS["1.5b-ttft"]
    print("bench: %s" % cfg["name"], file=sys.stderr, flush=True)
    tt = run_ttft(cfg, steps, warmup, stream)
    out["ttft_s8192"] = {"fused_over_vanilla": round(tt["fused"]["ms"] / tt["vanilla"]["ms"], 3),
                         "fused_ms": round(tt["fused"]["ms"], 4), "vanilla_ms": round(tt["vanilla"]["ms"], 4)}
    cfg = WORKLOADS["hgqa-decode"]
    print("bench: %s" % cfg["name"], file=sys.stderr, flush=True)
    hg, base = run_decode(cfg, steps, warmup, stream, variants=("fused",), graphs=False)
    del base
    torch.cuda.empty_cache()
    out["hgqa_g64_decode"] = {"frac": round(hg["fused"]["launch_rate"] / HBM_PEAK_GBS, 4),
                              "GB/s": round(hg["fused"]["launch_rate"], 2),
                              "avg_launch_us": round(hg["fused"]["launch"]["mean_ms"] * 1e3, 2)}
    cfg = WORKLOADS["kivi-decode"]
    print("bench: %s" % cfg["name"], file=sys.stderr, flush=True)
    kv = run_kivi(cfg, steps, warmup, stream, variants=("fused",))
    torch.cuda.empty_cache()
    out["kivi4_decode"] = {"frac": round(kv["fused"]["launch_rate"] / HBM_PEAK_GBS, 4),
                           "GB/s": round(kv["fused"]["launch_rate"], 2),
                           "avg_launch_us": round(kv["fused"]["launch"]["mean_ms"] * 1e3, 2),
                           "traffic": recorded_traffic("kivi")}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed repetitions (median, p10, p90 reported)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--part", choices=["all", "decode", "prefill", "next"], default="all")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=None,
                    help="measure one other configured workload instead of the default step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clocks", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run a plain float32 copy kernel over BYTES bytes (reads BYTES, writes BYTES), "
                         "used to scale the FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each GPU would run its own "
              "share of batch rows or KV heads with no exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    sampler = None if args.no_clocks else start_clock_sampler()
    try:
        import torch
        from cross_layer_kv_amd import binding
        binding.load_library()
        torch.cuda.set_device(0)
        stream = torch.cuda.current_stream()

        line = {"metric": "fused-KV decode attn HBM GB/s (% peak); prefill TFLOP/s (% MFMA) at S=8k",
                "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded N(0,1) post-RoPE caches, N(0.5,0.25) tied fusion weights)"}
        if args.workload:
            other_workload(args, line, stream)
        else:
            default_step(args, line, stream)
        copy_calibration(args, line)
    finally:
        clocks = stop_clock_sampler(sampler) if sampler is not None else {"clocks": "not sampled (--no-clocks)"}
    finish(line, clocks)


def default_step(args, line, stream):
    import torch
    dec = None
    if args.part in ("all", "decode"):
        print("bench: decode %s" % DECODE["name"], file=sys.stderr, flush=True)
        dec, base = run_decode(DECODE, args.steps, args.warmup, stream)
        f = dec["fused"]
        line.update(value=round(f["rate"], 2), ms_per_step=round(f["ms_per_step"], 4),
                    timing=dict(_stats_out(f["step"]), statistic="value and ms_per_step use the median step"))
        line["config"] = {"workload": DECODE["name"], "batch": DECODE["B"], "seq_len": DECODE["S"],
                          "q_heads": DECODE["Hq"], "kv_heads": DECODE["Hkv"], "head_dim": DECODE["D"],
                          "layers_per_step": DECODE["layers"], "cache_layout": "head-major [B,Hkv,S,D]",
                          "parallelism": "single GPU"}
        line["roofline"] = _hbm_roofline(f, "decode_kernel<bf16,96,fused,G=2>", recorded_traffic("decode"))
        line["decode_variants"] = _decode_block(dec)
        line["decode_variants"]["fused_over_vanilla_time"] = round(dec["fused"]["ms_per_layer"] /
                                                                   dec["vanilla"]["ms_per_layer"], 3)
        if not args.no_cpu_baseline:
            print("bench: cpu baseline (oracle, decode)", file=sys.stderr, flush=True)
            line["cpu_baseline"] = cpu_baseline(DECODE, base)
        del base
        torch.cuda.empty_cache()
    if args.part in ("all", "prefill"):
        print("bench: prefill %s" % PREFILL["name"], file=sys.stderr, flush=True)
        pre, base = run_prefill(PREFILL, args.steps, args.warmup, stream, keep_base=not args.no_cpu_baseline)
        fl = prefill_flops(PREFILL["B"], PREFILL["S"], PREFILL["Hq"], PREFILL["D"])
        blk = {"workload": PREFILL["name"], "batch": PREFILL["B"], "seq_len": PREFILL["S"],
               "q_heads": PREFILL["Hq"], "kv_heads": PREFILL["Hkv"], "head_dim": PREFILL["D"],
               "flops_per_layer": fl, "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
               "fusion": "in-kernel: every workgroup fuses the tiles it reads; nothing staged in memory"}
        for k, v in pre.items():
            blk[k] = {"TFLOP/s": round(v["rate"], 2), "ms_per_layer": round(v["ms_per_layer"], 4),
                      "frac": round(v["rate"] / MFMA_BF16_PEAK_TFLOPS, 4), "step": _stats_out(v["step"])}
        blk["roofline"] = _mfma_roofline(pre["fused"], "prefill_kernel<128,fused,G=2>", fl,
                                         recorded_traffic("prefill"))
        if base is not None:
            print("bench: cpu baseline (oracle, prefill)", file=sys.stderr, flush=True)
            blk["cpu_baseline"] = cpu_baseline_prefill(PREFILL, base)
            del base
            torch.cuda.empty_cache()
        line["prefill"] = blk
        if dec is None:
            f = pre["fused"]
            line.update(value=round(f["rate"], 2), unit="TFLOP/s", ms_per_step=round(f["ms_per_step"], 4),
                        config={"workload": PREFILL["name"]}, roofline=blk["roofline"],
                        timing=dict(_stats_out(f["step"]), statistic="value and ms_per_step use the median step"))
            if "cpu_baseline" in blk:
                line["cpu_baseline"] = blk["cpu_baseline"]
    if args.part in ("all", "next"):
        line["next_rows"] = next_rows(args.steps, args.warmup, stream)
        if dec is None and "value" not in line:
            s1 = line["next_rows"]["stack_b1_s131072"]
            line.update(value=s1["fused_ms"], unit="ms", higher_is_better=False, ms_per_step=s1["fused_ms"],
                        metric="whole-stack decode step time (ms), B=1, S=131072",
                        config={"workload": WORKLOADS["long-decode-b1"]["name"]})


def copy_calibration(args, line):
    """A plain float32 copy of args.copy_calibration bytes, for scaling the
    FETCH_SIZE / WRITE_SIZE counters of a profiler run of the same program."""
    if not args.copy_calibration:
        return
    import torch
    n = args.copy_calibration // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    line["copy_calibration_bytes"] = n * 4
    del src, dst


def finish(line, clocks):
    import torch
    props = torch.cuda.get_device_properties(0)
    line["device"] = {"name": props.name, "compute_units": props.multi_processor_count,
                      "arch": getattr(props, "gcnArchName", ""), "hip": torch.version.hip}
    line["device"].update(clocks)
    print(json.dumps(line), flush=True)


def other_workload(args, line, stream):
    cfg = WORKLOADS[args.workload]
    kind = cfg["kind"]
    print("bench: %s" % cfg["name"], file=sys.stderr, flush=True)
    shape = {"workload": cfg["name"], "batch": cfg["B"], "seq_len": cfg["S"], "q_heads": cfg["Hq"],
             "kv_heads": cfg["Hkv"], "head_dim": cfg["D"]}
    med = "value and ms_per_step use the median step"
    if kind == "decode":
        res, _ = run_decode(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        line.update(value=round(f["rate"], 2), ms_per_step=round(f["ms_per_step"], 4),
                    dtype="f32" if cfg.get("dtype") == "f32" else "bf16",
                    config=dict(shape, layers_per_step=cfg["layers"]),
                    timing=dict(_stats_out(f["step"]), statistic=med))
        line["roofline"] = _hbm_roofline(f, "fused decode", None)
        line["decode_variants"] = _decode_block(res)
        line["decode_variants"]["fused_over_vanilla_time"] = round(res["fused"]["ms_per_layer"] /
                                                                   res["vanilla"]["ms_per_layer"], 3)
    elif kind == "prefill":
        res, _ = run_prefill(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        fl = prefill_flops(cfg["B"], cfg["S"], cfg["Hq"], cfg["D"])
        line.update(value=round(f["rate"], 2), unit="TFLOP/s", ms_per_step=round(f["ms_per_step"], 4),
                    metric="fused-KV causal prefill TFLOP/s (% MFMA)",
                    config=dict(shape, layers_per_step=cfg["layers"]),
                    timing=dict(_stats_out(f["step"]), statistic=med))
        line["roofline"] = _mfma_roofline(f, "fused prefill (in-kernel fusion)", fl)
        line["prefill_variants"] = {k: {"TFLOP/s": round(v["rate"], 2), "ms_per_layer": round(v["ms_per_layer"], 4),
                                        "frac": round(v["rate"] / MFMA_BF16_PEAK_TFLOPS, 4),
                                        "step": _stats_out(v["step"])} for k, v in res.items()}
    elif kind == "stack":
        res = run_stack(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        line.update(value=round(f["gbs"], 2), ms_per_step=round(f["ms_per_step"], 4),
                    metric="whole-stack decode attention HBM GB/s (% peak)",
                    config=dict(shape, layers=2 * cfg["layers"]),
                    timing=dict(_stats_out(f["step"]), statistic=med + " (HIP-graph replay)"))
        line["roofline"] = {"bound": "hbm", "achieved": round(f["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(f["gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                            "note": "whole step (24 launches) over its algorithmic bytes"}
        line["stack"] = {k: {"ms": round(v["ms_per_step"], 4), "GB/s": round(v["gbs"], 2), "bytes": v["bytes"],
                             "graph_step": _stats_out(v["step"]), "eager_step": _stats_out(v["eager"])}
                         for k, v in res.items()}
        line["stack"]["time_over_vanilla"] = {k: round(res[k]["ms_per_step"] / res["vanilla"]["ms_per_step"], 3)
                                              for k in ("fused", "lite")}
        line["stack"]["bytes_over_vanilla"] = {k: round(res[k]["bytes"] / res["vanilla"]["bytes"], 3)
                                               for k in ("fused", "lite")}
    elif kind == "backward":
        res = run_backward(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        fl = backward_flops(cfg["B"], cfg["S"], cfg["Hq"], cfg["D"])
        line.update(value=round(f["rate"], 2), unit="TFLOP/s", ms_per_step=round(f["ms_per_step"], 4),
                    metric="fused-KV causal prefill backward TFLOP/s (% MFMA)",
                    config=dict(shape, layers_per_step=cfg["layers"]),
                    timing=dict(_stats_out(f["step"]), statistic=med))
        line["roofline"] = {"bound": "mfma", "achieved": round(f["rate"], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(f["rate"] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                            "flops_per_launch": fl, "avg_call_ms": round(f["ms_per_layer"], 4),
                            "note": "per call (prep, key-tile, query-tile and reduce kernels) at the median step"}
        line["backward_variants"] = {k: {"TFLOP/s": round(v["rate"], 2), "ms_per_layer": round(v["ms_per_layer"], 4),
                                         "frac": round(v["rate"] / MFMA_BF16_PEAK_TFLOPS, 4),
                                         "step": _stats_out(v["step"])} for k, v in res.items()}
    elif kind == "kivi":
        res = run_kivi(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        line.update(value=round(f["rate"], 2), ms_per_step=round(f["ms_per_step"], 4),
                    metric="4-bit fused-KV decode HBM GB/s (% peak)", config=dict(shape, layers_per_step=cfg["layers"]),
                    timing=dict(_stats_out(f["step"]), statistic=med))
        line["roofline"] = _hbm_roofline(f, "q4_decode_kernel<96,fused,G=2>", recorded_traffic("kivi"))
        line["kivi"] = {k: {"GB/s": round(v["rate"], 2), "us_per_layer": round(v["ms_per_layer"] * 1e3, 2),
                            "frac": round(v["rate"] / HBM_PEAK_GBS, 4), "step": _stats_out(v["step"])}
                        for k, v in res.items() if k != "quantise"}
        line["kivi"]["bf16_over_4bit_time"] = round(res["bf16_fused"]["ms_per_layer"] / f["ms_per_layer"], 3)
        line["kivi"]["quantise"] = {"us_per_source": round(res["quantise"]["ms_per_source"] * 1e3, 2),
                                    "bf16_read_GB/s": round(res["quantise"]["gbs"], 2)}
    else:  # ttft
        res = run_ttft(cfg, args.steps, args.warmup, stream)
        line.update(value=round(res["fused"]["ms"], 4), unit="ms", higher_is_better=False,
                    metric="attention time to first token (ms), FusedKV schedule",
                    ms_per_step=round(res["fused"]["ms"], 4), config=dict(shape, layers=2 * cfg["layers"]),
                    timing=dict(_stats_out(res["fused"]["step"]), statistic=med))
        line["ttft"] = {"fused_ms": round(res["fused"]["ms"], 4), "vanilla_ms": round(res["vanilla"]["ms"], 4),
                        "fused_over_vanilla": round(res["fused"]["ms"] / res["vanilla"]["ms"], 3),
                        "fused_step": _stats_out(res["fused"]["step"]),
                        "vanilla_step": _stats_out(res["vanilla"]["step"])}


if __name__ == "__main__":
    main()
