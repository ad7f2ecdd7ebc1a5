"""GPU parity of fkv_decode / fkv_lite_decode against the fp64 oracle, through
the C ABI.  Every test prints its case before touching the GPU."""
import os

import numpy as np
import pytest
import torch

from cross_layer_kv_amd import binding, inputs
from parity import TOL, gpu_rows, lse_err, oracle_layer, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_decode(L, fused=True, single=("kn", "v1"), ws=None):
    B, _, Hq, D = L.q.shape
    out = torch.full_like(L.q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    if ws is None:
        ws = binding.decode_workspace(L.q, L.k1)
    if fused:
        binding.fkv_decode(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, out=out, lse=lse, workspace=ws,
                           seqlens_k=L.seqlens_k)
    else:
        binding.fkv_lite_decode(L.q, getattr(L, single[0]), getattr(L, single[1]), out=out, lse=lse,
                                workspace=ws, seqlens_k=L.seqlens_k)
    torch.cuda.synchronize()
    return out, lse


def check(L, fused=True, single=("kn", "v1"), tol=None):
    B, _, Hq, D = L.q.shape
    out, lse = run_decode(L, fused, single)
    ro, rl = oracle_layer(L, fused=fused, single=single)
    tol = tol or TOL[L.q.dtype]
    e = rel_err(gpu_rows(out, B, Hq, 1, D), ro)
    el = lse_err(lse.cpu().numpy().reshape(-1), rl)
    say("  err=%.3e lse_err=%.3e tol=%.0e" % (e, el, tol))
    assert e <= tol and el <= tol, (e, el)
    return out, lse


def test_tiny_fp32_config_fused_and_lite():
    """Tiny decode: B=1, S=1024, Hq=4, Hkv=2, D=64, fp32, FusedKV and Lite."""
    say("decode tiny fp32 B=1 S=1024 Hq=4 Hkv=2 D=64 seed=0xF0001")
    L = inputs.make_layer(1, 1, 1024, 4, 2, 64, torch.float32, 0xF0001, DEV)
    check(L, fused=True)
    check(L, fused=False)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 80, 96, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_head_dims_and_gqa_ratios(dtype, D, G):
    Hkv = 2
    say("decode sweep dtype=%s D=%d G=%d B=2 S=333" % (dtype, D, G))
    L = inputs.make_layer(2, 1, 333, Hkv * G, Hkv, D, dtype, 100 + D + G, DEV)
    check(L, fused=True)
    check(L, fused=False)


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_layouts_and_ragged_lengths(layout):
    say("decode layout=%s ragged seqlens" % layout)
    L = inputs.make_layer(5, 1, 517, 16, 8, 96, torch.bfloat16, 7, DEV, layout=layout,
                          seqlens_k=[517, 1, 0, 64, 300])
    out, lse = check(L, fused=True)
    # the empty row: O = 0 and LSE = -inf exactly
    assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))
    check(L, fused=False)


def test_empty_cache():
    say("decode seqlen_k=0")
    L = inputs.make_layer(2, 1, 0, 4, 2, 64, torch.bfloat16, 9, DEV)
    out, lse = run_decode(L)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_forced_split_counts(splits, monkeypatch):
    monkeypatch.setenv("FKV_DECODE_SPLITS", str(splits))
    say("decode forced splits=%d" % splits)
    L = inputs.make_layer(2, 1, 4100, 8, 4, 128, torch.bfloat16, 11, DEV)
    check(L, fused=True)
    check(L, fused=False)


def test_selector_weights_match_lite(monkeypatch):
    """(a, a', b, b') = (0, 1, 1, 0) makes the fused kernel read exactly K^n
    and V^1 ([Deck] frame "Lite separates the key source from the value
    source", Eq. (6)).  The two kernels split the tokens over different wave
    counts, so they agree up to float32 summation order: O within one bf16
    rounding, LSE within 1e-5; both also match the oracle."""
    monkeypatch.setenv("FKV_DECODE_SPLITS", "5")
    say("decode selector weights vs lite")
    L = inputs.make_layer(3, 1, 1000, 8, 4, 80, torch.bfloat16, 12, DEV)
    z = torch.zeros_like(L.weights[0])
    o = torch.ones_like(L.weights[0])
    L.weights = (z, o, o, z)
    of, lf = check(L, fused=True)
    ol, ll = check(L, fused=False, single=("kn", "v1"))
    B, _, Hq, D = L.q.shape
    assert rel_err(gpu_rows(of, B, Hq, 1, D), gpu_rows(ol, B, Hq, 1, D)) <= 2 ** -8
    assert lse_err(lf.cpu().numpy(), ll.cpu().numpy()) <= 1e-5


def test_workspace_reuse_is_deterministic(monkeypatch):
    """Repeated calls on one workspace (split path and direct path) give
    identical results; the workspace needs no initialisation."""
    say("decode repeated calls on one workspace")
    L = inputs.make_layer(4, 1, 2000, 16, 8, 128, torch.bfloat16, 13, DEV)
    for splits in ("5", "1"):
        monkeypatch.setenv("FKV_DECODE_SPLITS", splits)
        ws = torch.full((max(256, binding.fkv_decode_workspace_size(binding.make_params(L.q, L.k1))),),
                        255, dtype=torch.uint8, device=DEV)   # garbage on purpose
        a = run_decode(L, ws=ws)
        b = run_decode(L, ws=ws)
        c = run_decode(L, fused=False, ws=ws)
        d = run_decode(L, ws=ws)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[0], d[0])
        assert not torch.equal(a[0], c[0])


def test_vanilla_control_on_own_caches():
    """Plain storage-layer attention: the single-source kernel over (K^1, V^1)."""
    say("decode vanilla control (K1, V1)")
    L = inputs.make_layer(2, 1, 700, 16, 8, 128, torch.bfloat16, 14, DEV)
    check(L, fused=False, single=("k1", "v1"))


def _sampled(B, S, Hq, Hkv, D, seed, n_batches=2, n_heads=None, layers=1):
    say("decode full size B=%d S=%d Hq=%d Hkv=%d D=%d seed=%#x (sampled rows)" % (B, S, Hq, Hkv, D, seed))
    L = inputs.make_layer(B, 1, S, Hq, Hkv, D, torch.bfloat16, seed, DEV)
    rng = np.random.default_rng(seed)
    bs = sorted(set([0, B - 1] + list(rng.integers(0, B, size=max(0, n_batches - 2)))))
    for fused in (True, False):
        out, lse = run_decode(L, fused=fused)
        ro, rl = oracle_layer(L, fused=fused, batch=bs)
        got = gpu_rows(out[bs], len(bs), Hq, 1, D)
        e = rel_err(got, ro)
        el = lse_err(lse[bs].cpu().numpy().reshape(-1), rl)
        say("  fused=%s batches=%s err=%.3e lse_err=%.3e" % (fused, bs, e, el))
        assert e <= 1e-2 and el <= 1e-2
        # every row finite
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    del L
    torch.cuda.empty_cache()


def test_full_size_650m_decode():
    """650M shape: B=32, S=8192, 16/8 heads, D=96, bf16 (the benchmarked
    launch configuration); oracle on every head of sampled batch rows."""
    _sampled(32, 8192, 16, 8, 96, 0xF0002, n_batches=3)


def test_full_size_4b_decode():
    """4B shape: B=16, S=32768, 32/16 heads, D=80."""
    _sampled(16, 32768, 32, 16, 80, 0xF0004, n_batches=2)


@pytest.mark.parametrize("B", [1, 8])
def test_full_size_long_context_decode(B):
    """Long context: S=131072, 16/8 heads, D=128, batch 1 and 8."""
    _sampled(B, 131072, 16, 8, 128, 0xF0005, n_batches=2)


# ---- high GQA ratio: 64 query heads per KV head (matrix-core kernel) ----

@pytest.mark.parametrize("D", [64, 80, 96, 128])
def test_high_gqa_head_dims(D):
    """G = 64 ([Deck] frame "Decode cost depends on the inference regime",
    Fig. 5 right): 128 query heads over 2 KV heads, ragged tile tail."""
    say("decode high-GQA D=%d B=2 S=333 Hq=128 Hkv=2" % D)
    L = inputs.make_layer(2, 1, 333, 128, 2, D, torch.bfloat16, 900 + D, DEV)
    check(L, fused=True)
    check(L, fused=False)


@pytest.mark.parametrize("splits", [1, 3, 17])
def test_high_gqa_splits_and_ragged(splits, monkeypatch):
    """Forced split counts (1: direct write, else partials + merge) with
    ragged lengths, including an empty sequence and a single token."""
    monkeypatch.setenv("FKV_DECODE_SPLITS", str(splits))
    say("decode high-GQA splits=%d ragged seqlens" % splits)
    L = inputs.make_layer(4, 1, 2100, 64, 1, 128, torch.bfloat16, 950 + splits, DEV,
                          seqlens_k=[2100, 0, 1, 777])
    out, lse = check(L, fused=True)
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))
    check(L, fused=False)


@pytest.mark.parametrize("D", [80, 128])
def test_high_gqa_reference_max_raised_mid_sequence(D, monkeypatch):
    """One split over the whole cache; keys of the first 64-token tile
    scaled by 0.05 and later keys by 3, so for many heads the second tile's
    max exceeds the running max by more than 8 log2 units and the lazy
    rescale runs after a non-empty first tile."""
    monkeypatch.setenv("FKV_DECODE_SPLITS", "1")
    say("decode high-GQA mid-sequence max raises D=%d S=333" % D)
    S = 333
    L = inputs.make_layer(2, 1, S, 128, 2, D, torch.bfloat16, 970 + D, DEV)
    ramp = torch.where(torch.arange(S, device=DEV) < 64, 0.05, 3.0).to(torch.bfloat16).view(1, S, 1, 1)
    for t in (L.k1, L.kn):
        t.mul_(ramp)
    check(L, fused=True)
    check(L, fused=False)


@pytest.mark.xfail(reason="binary16 operand limit: scores near 100 log2 units carry ~2^-11 relative rounding "
                          "of the fused keys and the queries, which moves exponents by ~0.05 and the output by "
                          "2-3e-2; documented with fkv_decode for 64 query heads per KV head", strict=False)
@pytest.mark.parametrize("D", [80, 128])
def test_high_gqa_wide_score_range_binary16_limit(D, monkeypatch):
    """Keys of 64-token tile j scaled by (1 + 3j) over five tiles (scores near
    100 log2 units): the binary16 operand limit of the matrix-core decode,
    kept as an expected failure with its measured error."""
    monkeypatch.setenv("FKV_DECODE_SPLITS", "1")
    say("decode high-GQA wide score range (keys x(1+3j) per tile) D=%d S=320" % D)
    S = 320
    L = inputs.make_layer(2, 1, S, 128, 2, D, torch.bfloat16, 980 + D, DEV)
    ramp = (1.0 + 3.0 * (torch.arange(S, device=DEV) // 64).float()).to(torch.bfloat16).view(1, S, 1, 1)
    for t in (L.k1, L.kn):
        t.mul_(ramp)
    out, lse = run_decode(L, fused=True)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    ro, rl = oracle_layer(L, fused=True)
    e = rel_err(gpu_rows(out, 2, 128, 1, D), ro)
    el = lse_err(lse.cpu().numpy().reshape(-1), rl)
    say("  err=%.3e lse_err=%.3e" % (e, el))
    assert e <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16], (e, el)


def test_high_gqa_selector_weights_match_lite():
    """(a, a', b, b') = (0, 1, 1, 0): the fused kernel reads exactly K^n and
    V^1 and its fp16 tiles equal the Lite kernel's, bit for bit."""
    say("decode high-GQA selector weights vs lite")
    L = inputs.make_layer(2, 1, 1000, 128, 2, 80, torch.bfloat16, 960, DEV)
    z = torch.zeros_like(L.weights[0])
    o = torch.ones_like(L.weights[0])
    L.weights = (z, o, o, z)
    of, lf = run_decode(L, fused=True)
    ol, ll = run_decode(L, fused=False)
    assert torch.equal(of, ol) and torch.equal(lf, ll)


def test_full_size_high_gqa_decode():
    """High-GQA shape: B=16, S=32768, 128/2 heads, D=128 (the benchmarked
    launch); oracle on every head of sampled batch rows."""
    _sampled(16, 32768, 128, 2, 128, 0xF0006, n_batches=2)


def test_stack_graph_replay_matches_eager():
    """A decode stack (two storage-layer calls, a FusedKV call and a Lite call,
    all with the key axis split, so each call is two kernels over a shared
    workspace, then a FusedKV call on the matrix-core kernel for 64 query
    heads per KV head) captured as one HIP graph, as the bench replays steps.
    Every replay, with eager work and synchronisation between replays, equals
    the eager result bit for bit, and the FusedKV output matches the oracle."""
    B, S, Hq, Hkv, D = 1, 700, 8, 4, 96
    say("decode stack graph replay B=%d S=%d Hq=%d Hkv=%d D=%d bf16, plus G=64 D=128" % (B, S, Hq, Hkv, D))
    L = inputs.make_layer(B, 1, S, Hq, Hkv, D, torch.bfloat16, 0xF00D, DEV)
    H = inputs.make_layer(1, 1, 700, 128, 2, 128, torch.bfloat16, 0xF00E, DEV)  # matrix-core decode
    ws = binding.decode_workspace(L.q, L.k1)
    wsh = binding.decode_workspace(H.q, H.k1)
    outs = [torch.empty_like(L.q) for _ in range(4)] + [torch.empty_like(H.q)]

    def stack(st):
        binding.fkv_lite_decode(L.q, L.k1, L.v1, out=outs[0], workspace=ws, stream=st)
        binding.fkv_lite_decode(L.q, L.kn, L.vn, out=outs[1], workspace=ws, stream=st)
        binding.fkv_decode(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, out=outs[2], workspace=ws, stream=st)
        binding.fkv_lite_decode(L.q, L.kn, L.v1, out=outs[3], workspace=ws, stream=st)
        binding.fkv_decode(H.q, H.k1, H.kn, H.v1, H.vn, H.weights, out=outs[4], workspace=wsh, stream=st)

    stack(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    ro, _ = oracle_layer(L, fused=True)
    e = rel_err(gpu_rows(ref[2], B, Hq, 1, D), ro)
    ro, _ = oracle_layer(H, fused=True)
    eh = rel_err(gpu_rows(ref[4], 1, 128, 1, 128), ro)
    say("  eager fused err=%.3e, G=64 err=%.3e" % (e, eh))
    assert e <= TOL[torch.bfloat16] and eh <= TOL[torch.bfloat16]

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        stack(cap)
    cap.synchronize()
    with torch.cuda.graph(g, stream=cap):
        stack(cap)
    torch.cuda.synchronize()
    other = torch.empty_like(L.q)
    for r in range(4):
        for o in outs:
            o.fill_(float("nan"))
        # eager library work between replays, on the same workspace
        binding.fkv_decode(L.q, L.kn, L.k1, L.vn, L.v1, L.weights, out=other, workspace=ws)
        torch.cuda.synchronize()
        say("  replay %d" % r)
        g.replay()
        torch.cuda.synchronize()
        for i, (o, x) in enumerate(zip(outs, ref)):
            assert torch.equal(o, x), (r, i)


# ---- post-RoPE fusion at long positions ([Deck] frame "Post-RoPE fusion
# needs paired key weights", Eqs. (7)-(8); [Notes] section 2.4) ----

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_tied_weights_shift_invariant_at_long_positions(pairing, dtype):
    """The same raw draws rotated at positions 0..S-1 (query at S-1) and at
    131072-S..131071 (query at 131071).  With tied key weights every fused
    score depends only on the query-key offset, so both decodes agree: in
    float32 to float32 rounding (within 1e-4), in bfloat16 up to what the
    different bf16 rounding of the rotated caches moves the oracle itself,
    plus the 1e-2 tolerance.  Untied weights add a term in the absolute
    position and the outputs move far apart.  Each GPU result is also checked
    against the oracle."""
    B, S, Hq, Hkv, D = 2, 1024, 16, 8, 128
    shift = 131072 - S
    say("decode tied-weight shift invariance pairing=%s dtype=%s B=%d S=%d D=%d shift=%d"
        % (pairing, dtype, B, S, D, shift))
    dev_gpu, dev_orc = {}, {}
    for tied in (True, False):
        outs, refs = [], []
        for pos0 in (0, shift):
            L = inputs.make_layer(B, 1, S, Hq, Hkv, D, dtype, 0x5EED, DEV, pairing=pairing, pos0=pos0,
                                  tied=tied)
            out, _ = check(L, fused=True)
            outs.append(gpu_rows(out, B, Hq, 1, D))
            refs.append(oracle_layer(L, fused=True)[0])
        dev_gpu[tied] = rel_err(outs[1], outs[0])
        dev_orc[tied] = rel_err(refs[1], refs[0])
        say("  tied=%s shifted-vs-unshifted gpu %.3e oracle %.3e" % (tied, dev_gpu[tied], dev_orc[tied]))
    if dtype == torch.float32:
        assert dev_gpu[True] <= 1e-4
    else:
        assert dev_gpu[True] <= dev_orc[True] + TOL[dtype]
    assert dev_gpu[False] >= 0.1 and dev_orc[False] >= 0.1


# ---- rows past a sequence's length are never read (or never reach a sum) ----

def _poison_tails(L, value):
    """Fill every cache row t >= seqlens_k[b] of every source with `value`,
    inside the tensors (the caches keep their shape and strides)."""
    sl = L.seqlens_k.cpu().tolist()
    for name in ("k1", "kn", "v1", "vn"):
        t = getattr(L, name)
        for b, n in enumerate(sl):
            t[b, n:].fill_(value)


@pytest.mark.parametrize("G,D,splits", [(2, 96, "1"), (2, 128, "7"), (8, 80, "3"), (64, 128, "1"), (64, 80, "5")])
def test_nan_rows_past_seqlens_are_ignored(G, D, splits, monkeypatch):
    """Ragged rows whose cache entries past seqlens_k hold NaN (and +inf in a
    second run): the result equals the run on clean caches bit for bit and
    matches the oracle, for FusedKV and Lite, direct and split paths, the
    G <= 8 kernel (predicated loads) and the 64-head matrix-core kernel
    (rows past the end read through the buffer range check)."""
    monkeypatch.setenv("FKV_DECODE_SPLITS", splits)
    Hkv = 2 if G == 64 else 4
    say("decode NaN tails G=%d D=%d splits=%s" % (G, D, splits))
    L = inputs.make_layer(4, 1, 700, G * Hkv, Hkv, D, torch.bfloat16, 1700 + G + D, DEV,
                          seqlens_k=[700, 0, 131, 64])
    clean = {f: run_decode(L, fused=f) for f in (True, False)}
    for value in (float("nan"), float("inf")):
        _poison_tails(L, value)
        for fused in (True, False):
            out, lse = run_decode(L, fused=fused)
            assert torch.equal(out, clean[fused][0]) and torch.equal(lse, clean[fused][1]), (value, fused)
    out, lse = check(L, fused=True)
    assert torch.isfinite(out).all()
