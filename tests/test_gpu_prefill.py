"""GPU parity of fkv_prefill / fkv_lite_prefill (bf16 MFMA) against the fp64
oracle, through the C ABI, with the tiles fused inside the attention kernel
(no workspace) and fused once into a workspace first.  Every test prints its
case before touching the GPU."""
import numpy as np
import pytest
import torch

from cross_layer_kv_amd import binding, inputs
from parity import gpu_rows, lse_err, oracle_layer, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


def poisoned_workspace(L):
    """A fuse-once workspace filled with NaN bytes, so that any position the
    first kernel fails to write (padding rows included) shows up."""
    ws = binding.prefill_workspace(L.q, L.k1)
    ws.fill_(0xFF)
    return ws


def run_prefill(L, fused=True, causal=True, single=("kn", "v1"), ws=False):
    B, S, Hq, D = L.q.shape
    out = torch.full_like(L.q, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV)
    w = poisoned_workspace(L) if ws is True else (None if ws is False or ws is None else ws)
    if fused:
        binding.fkv_prefill(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, out=out, lse=lse, causal=causal, workspace=w)
    else:
        binding.fkv_lite_prefill(L.q, getattr(L, single[0]), getattr(L, single[1]), out=out, lse=lse,
                                 causal=causal, workspace=w)
    torch.cuda.synchronize()
    return out, lse


def check(L, fused=True, causal=True, single=("kn", "v1"), both=True):
    """The oracle once; the kernel without a workspace and (both=True) with
    a fuse-once workspace."""
    B, S, Hq, D = L.q.shape
    ro, rl = oracle_layer(L, fused=fused, causal=causal, single=single)
    for ws in ((False, True) if both else (False,)):
        out, lse = run_prefill(L, fused, causal, single, ws=ws)
        e = rel_err(gpu_rows(out, B, Hq, S, D), ro)
        el = lse_err(lse.cpu().numpy().reshape(-1), rl)
        say("  fuse_once=%s err=%.3e lse_err=%.3e" % (ws, e, el))
        assert e <= TOL and el <= TOL, (ws, e, el)
    return out, lse


@pytest.mark.parametrize("D", [64, 80, 96, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_head_dims_and_gqa_ratios(D, G):
    say("prefill sweep D=%d G=%d B=1 S=200 causal" % (D, G))
    L = inputs.make_layer(1, 200, 200, 2 * G, 2, D, torch.bfloat16, 200 + D + G, DEV, decode=False)
    check(L, fused=True)
    check(L, fused=False)


@pytest.mark.parametrize("S", [1, 63, 64, 65, 130, 257, 600])
def test_ragged_lengths(S):
    say("prefill ragged S=%d D=128 G=2" % S)
    L = inputs.make_layer(2, S, S, 4, 2, 128, torch.bfloat16, 300 + S, DEV, decode=False)
    check(L, fused=True)
    check(L, fused=False)


@pytest.mark.parametrize("D", [80, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_reference_max_raised_mid_row(D, causal):
    """Keys of the first 64-key tile scaled by 0.05 and all later keys by 3:
    in about half of the rows the second tile's max exceeds the running max
    by more than 8 log2 units, so the accumulator rescale (and, at D <= 96,
    the re-base of the score chains on a non-zero reference) runs in the
    middle of a row.  Scores stay within ~30 log2 units: larger ones lose
    more than the tolerance to binary16 operand rounding in any form of the
    kernel (a CPU emulation of its roundings puts this case at 0.006-0.007)."""
    say("prefill mid-row max raises D=%d causal=%s S=320" % (D, causal))
    S = 320
    L = inputs.make_layer(1, S, S, 4, 2, D, torch.bfloat16, 500 + D, DEV, decode=False)
    ramp = torch.where(torch.arange(S, device=DEV) < 64, 0.05, 3.0).to(torch.bfloat16).view(1, S, 1, 1)
    for t in (L.k1, L.kn):
        t.mul_(ramp)
    check(L, fused=True, causal=causal)
    check(L, fused=False, causal=causal)


@pytest.mark.parametrize("D", [80, 128])
def test_non_causal(D):
    say("prefill non-causal D=%d S=190" % D)
    L = inputs.make_layer(1, 190, 190, 4, 2, D, torch.bfloat16, 400 + D, DEV, decode=False)
    check(L, fused=True, causal=False)
    check(L, fused=False, causal=False)


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_layouts(layout):
    say("prefill layout=%s" % layout)
    L = inputs.make_layer(2, 300, 300, 16, 8, 96, torch.bfloat16, 500, DEV, layout=layout, decode=False)
    check(L, fused=True)


@pytest.mark.parametrize("ws", [False, True])
def test_selector_weights_equal_lite_bitwise(ws):
    """(0, 1, 1, 0) weights give K~ = K^n and V~ = V^1 exactly (also after the
    binary16 rounding of the fused tiles), so the fused kernel must equal the
    Lite kernel bit for bit."""
    say("prefill selector weights vs lite fuse_once=%s" % ws)
    L = inputs.make_layer(1, 333, 333, 8, 4, 80, torch.bfloat16, 600, DEV, decode=False)
    z = torch.zeros_like(L.weights[0])
    o = torch.ones_like(L.weights[0])
    L.weights = (z, o, o, z)
    of, lf = run_prefill(L, fused=True, ws=ws)
    ol, ll = run_prefill(L, fused=False, ws=ws)
    assert torch.equal(of, ol) and torch.equal(lf, ll)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_fuse_once_single_source_equals_in_kernel_bitwise(D):
    """Single-source tiles convert from bf16 to binary16 exactly, so staging
    them once in the workspace or in the kernel gives the same operands and
    the same results bit for bit (S = 300 leaves a ragged last tile)."""
    say("prefill lite fuse-once vs in-kernel D=%d S=300 G=2" % D)
    L = inputs.make_layer(2, 300, 300, 8, 4, D, torch.bfloat16, 650 + D, DEV, decode=False)
    o0, l0 = run_prefill(L, fused=False, ws=False)
    o1, l1 = run_prefill(L, fused=False, ws=True)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_fuse_once_workspace_reused_for_a_smaller_prompt():
    """One workspace serves a call and then a call with a shorter prompt and
    fewer heads; the second call's tiles overwrite what it reads."""
    say("prefill fuse-once workspace reuse: S=520 Hkv=4 then S=130 Hkv=2 (D=96)")
    big = inputs.make_layer(1, 520, 520, 8, 4, 96, torch.bfloat16, 660, DEV, decode=False)
    ws = poisoned_workspace(big)
    for L in (big, inputs.make_layer(1, 130, 130, 4, 2, 96, torch.bfloat16, 661, DEV, decode=False)):
        B, S, Hq, D = L.q.shape
        out, lse = run_prefill(L, fused=True, ws=ws)
        ro, rl = oracle_layer(L, fused=True, causal=True)
        e = rel_err(gpu_rows(out, B, Hq, S, D), ro)
        el = lse_err(lse.cpu().numpy().reshape(-1), rl)
        say("  S=%d err=%.3e lse_err=%.3e" % (S, e, el))
        assert e <= TOL and el <= TOL


def test_vanilla_control_on_own_caches():
    say("prefill vanilla control (K1, V1)")
    L = inputs.make_layer(1, 257, 257, 16, 8, 128, torch.bfloat16, 700, DEV, decode=False)
    check(L, fused=False, single=("k1", "v1"))


def _sample_rows(B, Hq, S, bm, rng, per_bh=16):
    """Stratified rows: first/last rows, rows around tile boundaries and
    random rows for a few (b, h) pairs."""
    rows = []
    bhs = [(0, 0), (B - 1, Hq - 1), (int(rng.integers(B)), int(rng.integers(Hq)))]
    for b, h in bhs:
        ps = {0, 1, S - 1, S - 2}
        for t in range(bm, S, bm * 7):
            ps.update({t - 1, t})
        ps.update(int(x) for x in rng.integers(0, S, size=per_bh))
        rows += [(b * Hq + h) * S + p for p in sorted(ps) if 0 <= p < S]
    return np.array(sorted(set(rows)), dtype=np.int64)


def _full_size(B, S, Hq, Hkv, D, seed):
    say("prefill full size B=%d S=%d Hq=%d Hkv=%d D=%d seed=%#x (sampled rows)" % (B, S, Hq, Hkv, D, seed))
    L = inputs.make_layer(B, S, S, Hq, Hkv, D, torch.bfloat16, seed, DEV, decode=False)
    rng = np.random.default_rng(seed)
    rows = _sample_rows(B, Hq, S, 256 // (Hq // Hkv), rng)
    ws = binding.prefill_workspace(L.q, L.k1)
    for fused in (True, False):
        ro, rl = oracle_layer(L, fused=fused, causal=True, rows=rows)
        for w in (None, ws):
            if w is not None:
                w.fill_(0xFF)
            out, lse = run_prefill(L, fused=fused, ws=w if w is not None else False)
            assert torch.isfinite(out).all() and torch.isfinite(lse).all()
            got = gpu_rows(out, B, Hq, S, D)[rows]
            e = rel_err(got, ro)
            el = lse_err(lse.cpu().numpy().reshape(-1)[rows], rl)
            say("  fused=%s fuse_once=%s rows=%d err=%.3e lse_err=%.3e" % (fused, w is not None, rows.size, e, el))
            assert e <= TOL and el <= TOL
    del ws
    del L
    torch.cuda.empty_cache()


def test_full_size_1p5b_prefill():
    """1.5B shape: B=4, S=8192, 16/8 heads, D=128 (the benchmarked launch)."""
    _full_size(4, 8192, 16, 8, 128, 0xF0003)


def test_full_size_4b_prefill():
    """4B shape: B=1, S=16384, 32/16 heads, D=80."""
    _full_size(1, 16384, 32, 16, 80, 0xF0004)


@pytest.mark.parametrize("S", [200, 4100])
def test_first_token_row_equals_decode(S):
    """Time to first token needs only the final prompt position of a
    reconstruction layer.  Under the causal mask that row sees every cached
    token, so a decode with the same query (position S-1) over the S-token
    caches must reproduce the final prefill row and its LSE; both are checked
    against the oracle's causal row S-1 and against each other."""
    say("ttft: decode at S=%d vs causal prefill row S-1 (B=2 16/8 D=128)" % S)
    B, Hq, Hkv, D = 2, 16, 8, 128
    L = inputs.make_layer(B, S, S, Hq, Hkv, D, torch.bfloat16, 800 + S, DEV, decode=False)
    out_p, lse_p = run_prefill(L, fused=True)
    qlast = L.q[:, S - 1:S].contiguous()
    out_d = torch.full_like(qlast, float("nan"))
    lse_d = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    binding.fkv_decode(qlast, L.k1, L.kn, L.v1, L.vn, L.weights, out=out_d, lse=lse_d,
                       workspace=binding.decode_workspace(qlast, L.k1))
    torch.cuda.synchronize()
    rows = np.array([(b * Hq + h) * S + S - 1 for b in range(B) for h in range(Hq)], dtype=np.int64)
    ro, rl = oracle_layer(L, fused=True, causal=True, rows=rows)
    got_d = gpu_rows(out_d, B, Hq, 1, D)
    got_p = gpu_rows(out_p[:, S - 1:S], B, Hq, 1, D)
    e_d, e_p = rel_err(got_d, ro), rel_err(got_p, ro)
    el_d = lse_err(lse_d.cpu().numpy().reshape(-1), rl)
    el_p = lse_err(lse_p[:, :, S - 1].cpu().numpy().reshape(-1), rl)
    e_pd = rel_err(got_p, got_d)
    say("  decode err=%.3e lse=%.3e  prefill err=%.3e lse=%.3e  prefill-vs-decode %.3e"
        % (e_d, el_d, e_p, el_p, e_pd))
    assert e_d <= TOL and el_d <= TOL and e_p <= TOL and el_p <= TOL and e_pd <= TOL
