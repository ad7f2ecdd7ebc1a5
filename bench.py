"""Benchmark of FusedKV reconstruction-layer attention on one MI355X.

One step is one decode pass over every reconstruction layer of the 650M-shape
model (16 layers; layers 9..16 rebuild K/V from layers 1 and 8): 8 calls of
fkv_decode, batch 32, 8192 cached tokens, 16 query / 8 KV heads, head dim 96,
bf16, head-major caches, each layer with its own queries and fusion vectors.
`value` is the step's algorithmic cache traffic divided by its time (GB/s).
Beside it the line reports the causal prefill of the 1.5B shape (batch 4,
S = 8192, 16/8 heads, D = 128, 12 fused layers) in TFLOP/s, the Lite and
plain-control variants, the roofline of the decode kernel, and the fp64
oracle timed on the host cores on a bounded sample of the decode workload.

Algorithmic work (what the method must move or compute, per layer call):
  decode  bytes = 4*B*S*Hkv*D*2 (four bf16 source caches; 2 for Lite/vanilla)
                  + 2*B*Hq*D*2 (Q, O) + 16*Hkv*D (fp32 weights)
  prefill flops = 2*D*S*(S+1)*B*Hq (QK^T and PV over the causal triangle)
Inputs are synthetic and seeded (see cross_layer_kv_amd/inputs.py) and
resident in HBM before timing starts.

`--workload NAME` measures one of the other configured workloads instead and
prints one JSON line for it: tiny-decode (fp32, cache-resident correctness
shape), 4b-decode, hgqa-decode (64 query heads per KV head, matrix-core
kernel), 4b-prefill, 1.5b-prefill, long-decode-b1 / long-decode-b8
(131072 cached tokens; the whole 24-layer stack: 12 storage layers of plain
attention plus 12 reconstruction layers, FusedKV vs Lite vs an all-vanilla
model, each step replayed as one HIP graph, with the eager time beside it),
and 1.5b-ttft (time to first token over the attention of all 24
layers: the storage layers run causal prefill, the reconstruction layers only
the final query row, a decode at S, against 24 layers of causal prefill).
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


def decode_source_sha():
    """sha256[:16] over the decode kernel source and the header that sets its
    launch shape (waves per workgroup, tokens per wave step)."""
    h = hashlib.sha256()
    for name in ("fkv_decode.hip", "fkv_internal.h"):
        h.update(open(os.path.join(ROOT, "cross_layer_kv_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the four-source decode kernel, from the
    committed counter summary (FETCH_SIZE and WRITE_SIZE runs scaled by a
    copy kernel of known size); None when the kernel source has changed
    since the counters were taken, or when there is no summary."""
    path = os.path.join(ROOT, "profiles", "decode_650m_bf16_hbm_traffic.txt")
    try:
        text = open(path, encoding="utf-8").read()
        sha = decode_source_sha()
    except OSError:
        return None
    fields = {}
    for ln in text.splitlines():
        if ln and not ln.startswith("#") and ":" in ln:
            k, v = ln.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


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


def _time_region(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps  # ms per call of fn


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


def run_decode(cfg, steps, warmup, stream):
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

    def fused_step(st=stream):
        for i in range(nl):
            binding.fkv_decode(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], out=outs[i],
                               workspace=ws, stream=st)

    def lite_step(st=stream):
        for i in range(nl):
            binding.fkv_lite_decode(qs[i], base.kn, base.v1, out=outs[i], workspace=ws, stream=st)

    def vanilla_step(st=stream):  # storage-layer control: attention over a layer's own caches
        for i in range(nl):
            k, v = (base.k1, base.v1) if i % 2 == 0 else (base.kn, base.vn)
            binding.fkv_lite_decode(qs[i], k, v, out=outs[i], workspace=ws, stream=st)

    res = {}
    elt = 4 if dt == torch.float32 else 2
    for name, fn, src in (("fused", fused_step, 4), ("lite", lite_step, 2), ("vanilla", vanilla_step, 2)):
        ms = _time_region(fn, steps, warmup, stream)
        byts = decode_bytes(B, S, Hq, Hkv, D, src, elt) * nl
        # the same step replayed as one HIP graph: no host launch cost between kernels
        g = _capture(fn, stream)
        gms = _time_region(g.replay, steps, warmup, stream)
        del g
        res[name] = dict(ms_per_step=ms, ms_per_layer=ms / nl, gbs=byts / (ms * 1e-3) / 1e9,
                         bytes_per_layer=byts // nl, graph_ms_per_layer=gms / nl,
                         graph_gbs=byts / (gms * 1e-3) / 1e9)
    return res, base


def run_kivi(cfg, steps, warmup, stream):
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

    def fused_step():
        for i in range(nl):
            binding.fkv_kivi_decode(qs[i], q4["k1"], q4["kn"], q4["v1"], q4["vn"], ws_list[i], out=outs[i],
                                    workspace=ws, stream=stream)

    def lite_step():
        for i in range(nl):
            binding.fkv_kivi_lite_decode(qs[i], q4["kn"], q4["v1"], out=outs[i], workspace=ws, stream=stream)

    def bf16_step():
        for i in range(nl):
            binding.fkv_decode(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], out=outs[i],
                               workspace=ws, stream=stream)

    res = {}
    for name, fn, byts in (("fused", fused_step, kivi_decode_bytes(B, S, Hq, Hkv, D, 4) * nl),
                           ("lite", lite_step, kivi_decode_bytes(B, S, Hq, Hkv, D, 2) * nl),
                           ("bf16_fused", bf16_step, decode_bytes(B, S, Hq, Hkv, D, 4) * nl)):
        ms = _time_region(fn, steps, warmup, stream)
        res[name] = dict(ms_per_step=ms, ms_per_layer=ms / nl, gbs=byts / (ms * 1e-3) / 1e9,
                         bytes_per_layer=byts // nl)
    ms = _time_region(quantise_step, 2, 1, stream)
    res["quantise"] = dict(ms_per_source=ms / 4, gbs=B * S * Hkv * D * 2 / (ms / 4 * 1e-3) / 1e9)
    return res


def run_prefill(cfg, steps, warmup, stream):
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
    def fused_step():
        for i in range(nl):
            binding.fkv_prefill(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], out=out, causal=True,
                                stream=stream)

    def lite_step():
        for i in range(nl):
            binding.fkv_lite_prefill(qs[i], base.kn, base.v1, out=out, causal=True, stream=stream)

    res = {}
    fl = prefill_flops(B, S, Hq, D)
    for name, fn in (("fused", fused_step), ("lite", lite_step)):
        ms = _time_region(fn, max(1, steps // 2), max(1, warmup // 2), stream)
        res[name] = dict(ms_per_step=ms, ms_per_layer=ms / nl,
                         tflops=fl * nl / (ms * 1e-3) / 1e12)
    del qs, out, base
    torch.cuda.empty_cache()
    return res


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

    def fused_step():
        for i in range(nl):
            o, l = fwd["fused"][i]
            binding.fkv_prefill_backward(qs[i], base.k1, base.kn, base.v1, base.vn, ws_list[i], o, l, douts[i],
                                         dq=dq, dk1=grads[0], dkn=grads[1], dv1=grads[2], dvn=grads[3], dweights=dw,
                                         workspace=ws, causal=True, stream=stream)

    def lite_step():
        for i in range(nl):
            o, l = fwd["lite"][i]
            binding.fkv_lite_prefill_backward(qs[i], base.kn, base.v1, o, l, douts[i], dq=dq, dk=grads[0],
                                              dv=grads[2], workspace=ws, causal=True, stream=stream)

    res = {}
    fl = backward_flops(B, S, Hq, D)
    for name, fn in (("fused", fused_step), ("lite", lite_step)):
        ms = _time_region(fn, max(1, steps // 2), max(1, warmup // 2), stream)
        res[name] = dict(ms_per_step=ms, ms_per_layer=ms / nl, tflops=fl * nl / (ms * 1e-3) / 1e12)
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
        eager = _time_region(fn, steps, warmup, stream)
        # the whole step as one HIP graph, replayed on the timing stream
        g = _capture(fn, stream)
        ms = _time_region(g.replay, steps, warmup, stream)
        res[name] = dict(ms_per_step=ms, gbs=byts / (ms * 1e-3) / 1e9, bytes=byts, eager_ms_per_step=eager)
        del g
    return res


def run_ttft(cfg, steps, warmup, stream):
    """Attention time to first token of a 2n-layer model: storage layers run
    causal prefill over the prompt; FusedKV reconstruction layers need only
    the final prompt position, i.e. one decode at S per layer.  The plain
    model runs causal prefill in all 2n layers."""
    import torch
    from cross_layer_kv_amd import binding, inputs
    dev = "cuda:0"
    B, S, Hq, Hkv, D, nl = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["layers"]
    base = inputs.make_layer(B, S, S, Hq, Hkv, D, torch.bfloat16, cfg["seed"], dev, decode=False)
    qfull = base.q
    qlast = qfull[:, S - 1:S].contiguous()
    out_full = torch.empty_like(qfull)
    out_last = torch.empty_like(qlast)
    ws = binding.decode_workspace(qlast, base.k1)
    pairs = [(base.k1, base.v1), (base.kn, base.vn)]

    def vanilla_model():
        for i in range(2 * nl):
            k, v = pairs[i % 2]
            binding.fkv_lite_prefill(qfull, k, v, out=out_full, causal=True, stream=stream)

    def fused_model():
        for i in range(nl):
            k, v = pairs[i % 2]
            binding.fkv_lite_prefill(qfull, k, v, out=out_full, causal=True, stream=stream)
        for i in range(nl):
            binding.fkv_decode(qlast, base.k1, base.kn, base.v1, base.vn, base.weights, out=out_last,
                               workspace=ws, stream=stream)

    res = {}
    for name, fn in (("vanilla", vanilla_model), ("fused", fused_model)):
        res[name] = dict(ms=_time_region(fn, max(1, steps // 2), max(1, warmup // 2), stream))
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
    nb = B
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--part", choices=["all", "decode", "prefill"], default="all")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=None,
                    help="measure one other configured workload instead of the default step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run a plain float32 copy kernel over BYTES bytes (reads BYTES, writes BYTES), "
                         "used to scale the FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each GPU would run its own "
              "share of batch rows or KV heads with no exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

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
        return
    dec = None
    if args.part in ("all", "decode"):
        print("bench: decode %s" % DECODE["name"], file=sys.stderr, flush=True)
        dec, base = run_decode(DECODE, args.steps, args.warmup, stream)
        f = dec["fused"]
        line.update(value=round(f["gbs"], 2), ms_per_step=round(f["ms_per_step"], 4))
        line["config"] = {"workload": DECODE["name"], "batch": DECODE["B"], "seq_len": DECODE["S"],
                          "q_heads": DECODE["Hq"], "kv_heads": DECODE["Hkv"], "head_dim": DECODE["D"],
                          "layers_per_step": DECODE["layers"], "cache_layout": "head-major [B,Hkv,S,D]",
                          "parallelism": "single GPU"}
        line["roofline"] = {"bound": "hbm", "kernel": "decode_kernel<bf16,96,fused,G=2>",
                            "achieved": round(f["bytes_per_layer"] / (f["ms_per_layer"] * 1e-3) / 1e9, 2),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(f["bytes_per_layer"] / (f["ms_per_layer"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": recorded_traffic(),
                            "bytes_per_launch": f["bytes_per_layer"],
                            "avg_launch_us": round(f["ms_per_layer"] * 1e3, 2)}
        line["decode_variants"] = {k: {"GB/s": round(v["gbs"], 2), "us_per_layer": round(v["ms_per_layer"] * 1e3, 2),
                                       "frac": round(v["gbs"] / HBM_PEAK_GBS, 4),
                                       "graph_GB/s": round(v["graph_gbs"], 2),
                                       "graph_us_per_layer": round(v["graph_ms_per_layer"] * 1e3, 2)}
                                   for k, v in dec.items()}
        line["decode_variants"]["fused_over_vanilla_time"] = round(dec["fused"]["ms_per_layer"] /
                                                                   dec["vanilla"]["ms_per_layer"], 3)
        if not args.no_cpu_baseline:
            print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
            line["cpu_baseline"] = cpu_baseline(DECODE, base)
        del base
        torch.cuda.empty_cache()
    if args.part in ("all", "prefill"):
        print("bench: prefill %s" % PREFILL["name"], file=sys.stderr, flush=True)
        pre = run_prefill(PREFILL, args.steps, args.warmup, stream)
        line["prefill"] = {"workload": PREFILL["name"], "batch": PREFILL["B"], "seq_len": PREFILL["S"],
                           "q_heads": PREFILL["Hq"], "kv_heads": PREFILL["Hkv"], "head_dim": PREFILL["D"],
                           "flops_per_layer": prefill_flops(PREFILL["B"], PREFILL["S"], PREFILL["Hq"], PREFILL["D"]),
                           "peak_tflops": MFMA_BF16_PEAK_TFLOPS}
        for k, v in pre.items():
            line["prefill"][k] = {"TFLOP/s": round(v["tflops"], 2), "ms_per_layer": round(v["ms_per_layer"], 4),
                                  "frac": round(v["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)}
        if dec is None:
            line.update(value=round(pre["fused"]["tflops"], 2), unit="TFLOP/s",
                        ms_per_step=round(pre["fused"]["ms_per_step"], 4),
                        config={"workload": PREFILL["name"]})
    copy_calibration(args, line)
    finish(line)


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


def finish(line):
    import torch
    props = torch.cuda.get_device_properties(0)
    line["device"] = {"name": props.name, "compute_units": props.multi_processor_count,
                      "arch": getattr(props, "gcnArchName", ""), "hip": torch.version.hip}
    print(json.dumps(line), flush=True)


def other_workload(args, line, stream):
    cfg = WORKLOADS[args.workload]
    kind = cfg["kind"]
    print("bench: %s" % cfg["name"], file=sys.stderr, flush=True)
    shape = {"workload": cfg["name"], "batch": cfg["B"], "seq_len": cfg["S"], "q_heads": cfg["Hq"],
             "kv_heads": cfg["Hkv"], "head_dim": cfg["D"]}
    if kind == "decode":
        res, _ = run_decode(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        line.update(value=round(f["gbs"], 2), ms_per_step=round(f["ms_per_step"], 4),
                    dtype="f32" if cfg.get("dtype") == "f32" else "bf16",
                    config=dict(shape, layers_per_step=cfg["layers"]))
        line["roofline"] = {"bound": "hbm", "achieved": round(f["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(f["gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                            "bytes_per_launch": f["bytes_per_layer"], "avg_launch_us": round(f["ms_per_layer"] * 1e3, 2)}
        line["decode_variants"] = {k: {"GB/s": round(v["gbs"], 2), "us_per_layer": round(v["ms_per_layer"] * 1e3, 2),
                                       "frac": round(v["gbs"] / HBM_PEAK_GBS, 4),
                                       "graph_GB/s": round(v["graph_gbs"], 2),
                                       "graph_us_per_layer": round(v["graph_ms_per_layer"] * 1e3, 2)}
                                   for k, v in res.items()}
        line["decode_variants"]["fused_over_vanilla_time"] = round(res["fused"]["ms_per_layer"] /
                                                                   res["vanilla"]["ms_per_layer"], 3)
    elif kind == "prefill":
        res = run_prefill(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        line.update(value=round(f["tflops"], 2), unit="TFLOP/s", ms_per_step=round(f["ms_per_step"], 4),
                    metric="fused-KV causal prefill TFLOP/s (% MFMA)",
                    config=dict(shape, layers_per_step=cfg["layers"]))
        line["roofline"] = {"bound": "mfma", "achieved": round(f["tflops"], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(f["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                            "flops_per_launch": prefill_flops(cfg["B"], cfg["S"], cfg["Hq"], cfg["D"]),
                            "avg_launch_us": round(f["ms_per_layer"] * 1e3, 2)}
        line["prefill_variants"] = {k: {"TFLOP/s": round(v["tflops"], 2), "ms_per_layer": round(v["ms_per_layer"], 4),
                                        "frac": round(v["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)} for k, v in res.items()}
    elif kind == "stack":
        res = run_stack(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        line.update(value=round(f["gbs"], 2), ms_per_step=round(f["ms_per_step"], 4),
                    metric="whole-stack decode attention HBM GB/s (% peak)",
                    config=dict(shape, layers=2 * cfg["layers"]))
        line["roofline"] = {"bound": "hbm", "achieved": round(f["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(f["gbs"] / HBM_PEAK_GBS, 4), "traffic": None}
        line["stack"] = {k: {"ms": round(v["ms_per_step"], 4), "GB/s": round(v["gbs"], 2), "bytes": v["bytes"],
                             "eager_ms": round(v["eager_ms_per_step"], 4)}
                         for k, v in res.items()}
        line["stack"]["time_over_vanilla"] = {k: round(res[k]["ms_per_step"] / res["vanilla"]["ms_per_step"], 3)
                                              for k in ("fused", "lite")}
        line["stack"]["bytes_over_vanilla"] = {k: round(res[k]["bytes"] / res["vanilla"]["bytes"], 3)
                                               for k in ("fused", "lite")}
    elif kind == "backward":
        res = run_backward(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        line.update(value=round(f["tflops"], 2), unit="TFLOP/s", ms_per_step=round(f["ms_per_step"], 4),
                    metric="fused-KV causal prefill backward TFLOP/s (% MFMA)",
                    config=dict(shape, layers_per_step=cfg["layers"]))
        line["roofline"] = {"bound": "mfma", "achieved": round(f["tflops"], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(f["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                            "flops_per_launch": backward_flops(cfg["B"], cfg["S"], cfg["Hq"], cfg["D"]),
                            "avg_call_ms": round(f["ms_per_layer"], 4)}
        line["backward_variants"] = {k: {"TFLOP/s": round(v["tflops"], 2), "ms_per_layer": round(v["ms_per_layer"], 4),
                                         "frac": round(v["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)} for k, v in res.items()}
    elif kind == "kivi":
        res = run_kivi(cfg, args.steps, args.warmup, stream)
        f = res["fused"]
        line.update(value=round(f["gbs"], 2), ms_per_step=round(f["ms_per_step"], 4),
                    metric="4-bit fused-KV decode HBM GB/s (% peak)", config=dict(shape, layers_per_step=cfg["layers"]))
        line["roofline"] = {"bound": "hbm", "achieved": round(f["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(f["gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                            "bytes_per_launch": f["bytes_per_layer"], "avg_launch_us": round(f["ms_per_layer"] * 1e3, 2)}
        line["kivi"] = {k: {"GB/s": round(v["gbs"], 2), "us_per_layer": round(v["ms_per_layer"] * 1e3, 2),
                            "frac": round(v["gbs"] / HBM_PEAK_GBS, 4)} for k, v in res.items() if k != "quantise"}
        line["kivi"]["bf16_over_4bit_time"] = round(res["bf16_fused"]["ms_per_layer"] / f["ms_per_layer"], 3)
        line["kivi"]["quantise"] = {"us_per_source": round(res["quantise"]["ms_per_source"] * 1e3, 2),
                                    "bf16_read_GB/s": round(res["quantise"]["gbs"], 2)}
    else:  # ttft
        res = run_ttft(cfg, args.steps, args.warmup, stream)
        line.update(value=round(res["fused"]["ms"], 4), unit="ms", higher_is_better=False,
                    metric="attention time to first token (ms), FusedKV schedule",
                    ms_per_step=round(res["fused"]["ms"], 4), config=dict(shape, layers=2 * cfg["layers"]))
        line["ttft"] = {"fused_ms": round(res["fused"]["ms"], 4), "vanilla_ms": round(res["vanilla"]["ms"], 4),
                        "fused_over_vanilla": round(res["fused"]["ms"] / res["vanilla"]["ms"], 3)}
    copy_calibration(args, line)
    finish(line)


if __name__ == "__main__":
    main()
